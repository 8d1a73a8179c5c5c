// Merging normalised partial attention results by their log-sum-exp.
//
// Two partial results over disjoint key sets, (O_a, L_a) and (O_b, L_b), combine as
// L = log(e^{L_a} + e^{L_b}), O = e^{L_a - L} O_a + e^{L_b - L} O_b
// (page "LLM长文本推理Ring Attention环形注意力机制实现与优化", §Ring Attention实现代码
// 与通信重叠: the new lse and the two weights that rescale the old output and the
// block output). The n-way form is the reduction after split-KV partial attention
// (page "上下文并行 (CP) 收益评估实验设计", §Decode). Both are written max-shifted so
// that nothing overflows, and a -inf side contributes nothing.
//
// Both kernels are HBM-bound streams: one pass over the inputs, one over the outputs.
#include "common.hpp"

namespace ra {

// 2-way merge. A workgroup owns whole rows: it reads every row's two LSEs and
// derives the weights before any thread writes, so outputs may alias an input.
__global__ void __launch_bounds__(256)
lse_merge2_kernel(long long rows, int Dv, int rows_per_wg, const float* o_a, const float* lse_a,
                  const float* o_b, const float* lse_b, float* o_out, float* lse_out) {
  __shared__ float wa_s[256], wb_s[256], l_s[256];
  const long long row0 = (long long)blockIdx.x * rows_per_wg;
  const int nrows = (int)min((long long)rows_per_wg, rows - row0);
  const int t = threadIdx.x;
  if (t < nrows) {
    const float la = lse_a[row0 + t], lb = lse_b[row0 + t];
    const float mx = fmaxf(la, lb);
    float wa = 0.f, wb = 0.f, L = kNegInf;
    if (mx != kNegInf) {
      const float ea = exp2_hw((la - mx) * kLog2e), eb = exp2_hw((lb - mx) * kLog2e);
      const float tot = ea + eb;
      wa = ea / tot;
      wb = eb / tot;
      L = mx + log2_hw(tot) * kLn2;
    }
    wa_s[t] = wa;
    wb_s[t] = wb;
    l_s[t] = L;
  }
  __syncthreads();
  const int vec_per_row = Dv / 4;
  const int nvec = nrows * vec_per_row;
  const f32x4* A = (const f32x4*)(o_a + row0 * Dv);
  const f32x4* Bv = (const f32x4*)(o_b + row0 * Dv);
  f32x4* O = (f32x4*)(o_out + row0 * Dv);
  for (int e = t; e < nvec; e += 256) {
    const int r = e / vec_per_row;
    const f32x4 x = A[e], y = Bv[e];
    O[e] = wa_s[r] * x + wb_s[r] * y;
  }
  if (t < nrows) lse_out[row0 + t] = l_s[t];
}

// n-way merge: one wave per row. The wave reduces the partials' maximum LSE and
// exp-sum; each lane then streams its output columns, recomputing the n weights.
template <typename OutT>
__global__ void __launch_bounds__(256)
lse_merge_n_kernel(long long rows, int n, int Dv, const float* o_parts, const float* lse_parts,
                   OutT* o_out, float* lse_out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * 4 + wave;
  if (row >= rows) return;  // whole wave exits together; no barrier in this kernel
  const float* lp = lse_parts + row * n;
  float mx = kNegInf;
  for (int p = lane; p < n; p += 64) mx = fmaxf(mx, lp[p]);
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
  const float ms = mx == kNegInf ? 0.f : mx;
  float sum = 0.f;
  for (int p = lane; p < n; p += 64) sum += exp2_hw((lp[p] - ms) * kLog2e);
  for (int o = 32; o > 0; o >>= 1) sum += shfl_xor_f(sum, o);
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  const float* op = o_parts + row * (long long)n * Dv;
  for (int d = lane; d < Dv; d += 64) {
    float acc = 0.f;
    for (int p = 0; p < n; ++p)
      acc = fmaf(exp2_hw((lp[p] - ms) * kLog2e) * inv, op[(long long)p * Dv + d], acc);
    o_out[row * Dv + d] = (OutT)acc;
  }
  if (lane == 0) lse_out[row] = sum > 0.f ? ms + log2_hw(sum) * kLn2 : kNegInf;
}

hipError_t lse_merge2(long long rows, int Dv, const float* o_a, const float* lse_a, const float* o_b,
                      const float* lse_b, float* o_out, float* lse_out, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int rows_per_wg = max(1, min(256, 2048 / Dv));
  const long long grid = (rows + rows_per_wg - 1) / rows_per_wg;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lse_merge2_kernel, dim3((unsigned)grid), dim3(256), 0, st, rows, Dv, rows_per_wg,
                     o_a, lse_a, o_b, lse_b, o_out, lse_out);
  return hipGetLastError();
}

hipError_t lse_merge_n(int out_bf16, long long rows, int n, int Dv, const float* o_parts,
                       const float* lse_parts, void* o_out, float* lse_out, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const long long grid = (rows + 3) / 4;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (out_bf16)
    hipLaunchKernelGGL(lse_merge_n_kernel<__bf16>, dim3((unsigned)grid), dim3(256), 0, st, rows, n, Dv,
                       o_parts, lse_parts, (__bf16*)o_out, lse_out);
  else
    hipLaunchKernelGGL(lse_merge_n_kernel<float>, dim3((unsigned)grid), dim3(256), 0, st, rows, n, Dv,
                       o_parts, lse_parts, (float*)o_out, lse_out);
  return hipGetLastError();
}

}  // namespace ra
