// FP16 flash-attention path: the selective FP16 fallback of RotateAttention
// (arXiv 2607.02584, abstract) for masked heads, flagged Q/K blocks and whole
// denoising steps, with the log-sum-exp merge of mixed query blocks fused
// into its epilogue.
//
// Recurrences: RainFusion2.0, section 3.1 "Blockwise Sparse", in the log2
// domain over key blocks of 64; a tile that belongs to the INT4 path is
// skipped (the block mask M of the same section).
//
// Same work layout as the INT4 kernel: S^T = K Q^T and O^T = V^T P^T with
// v_mfma_f32_32x32x16_f16, one query column per lane, P rounded to fp16 in
// registers as the B operand of the second product, O accumulated in fp32
// by the matrix cores. Inputs are RoPE'd, unrotated Q/K (fp16, dense) and the
// caller's fp16 V. The V tile is transposed into LDS in the key order of
// the P operand so that each lane reads its operand with one 16-byte load.
#include "common.h"

namespace rotattn {

__device__ __forceinline__ float exp2_hw16(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D>
__global__ __launch_bounds__(256) void fp16_attn_kernel(KProblem kp, AttnArgs a, int whole_call, float c0) {
  constexpr int NC = D / 16;     // 16-deep slices per S tile (each lane half covers D/2 dims)
  constexpr int NCT = D / 32;
  constexpr int KP = D + 8;      // padded LDS row (halves)
  constexpr int VP = kBlock + 8;
  __shared__ __attribute__((aligned(16))) __half ks[kBlock * KP];
  __shared__ __attribute__((aligned(16))) __half vt[D * VP];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int L = kp.L, Lp = kp.Lp, NB = kp.NB;
  const int b = blockIdx.z, h = blockIdx.y, bh = b * kp.H + h;
  const int wrow = blockIdx.x * 128 + 32 * wave;
  const bool active = wrow < L;
  const int qblk = wrow / kBlock;
  bool full = false, mixed = false;
  if (active) {
    full = whole_call || (a.head_mask != nullptr && a.head_mask[bh] != 0) ||
           (a.route && a.q_flag[bh * NB + qblk] != 0);
    mixed = !full && a.route && a.head_kflag[bh] != 0;
  }
  const bool any_full = __syncthreads_or(full);
  const bool any_mixed = __syncthreads_or(mixed);
  if (!any_full && !any_mixed) return;

  const int row = wrow + col;
  v8h qop[NC];
  if (full || mixed) {
    const __half* qrow = a.q_rope + ((long long)bh * L + (row < L ? row : L - 1)) * D + hh * (D / 2);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint4 u = reinterpret_cast<const uint4*>(qrow)[c];
      qop[c] = *reinterpret_cast<const v8h*>(&u);
    }
  }

  float m_run = -INFINITY, l_part = 0.f;
  v16f o_acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int v = 0; v < 16; ++v) o_acc[ct][v] = 0.f;

  for (int j = 0; j < NB; ++j) {
    const bool kflag = a.route && a.k_flag[bh * NB + j] != 0;
    if (!any_full && !kflag) continue;
    __syncthreads();
    // K tile: 64 keys x D halves, rows at or beyond L are zero.
    for (int idx = threadIdx.x; idx < kBlock * D / 8; idx += 256) {
      const int r = idx / (D / 8), c8 = idx - r * (D / 8);
      const int key = j * kBlock + r;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (key < L) u = *reinterpret_cast<const uint4*>(a.k_rope + ((long long)bh * L + key) * D + c8 * 8);
      *reinterpret_cast<uint4*>(&ks[r * KP + c8 * 8]) = u;
    }
    // V tile, transposed: vt[channel][pos] with pos the operand order of key r.
    for (int idx = threadIdx.x; idx < kBlock * D / 8; idx += 256) {
      const int r = idx / (D / 8), c8 = idx - r * (D / 8);
      const int key = j * kBlock + r;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (key < L)
        u = *reinterpret_cast<const uint4*>(a.v + (long long)b * kp.sb + (long long)h * kp.sh +
                                            (long long)key * kp.sl + c8 * 8);
      const __half* hv = reinterpret_cast<const __half*>(&u);
      const int s = r >> 5, rr = r & 31;
      const int pos = 32 * s + 16 * (rr >> 4) + 8 * ((rr >> 2) & 1) + 4 * ((rr >> 3) & 1) + (rr & 3);
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[(c8 * 8 + e) * VP + pos] = hv[e];
    }
    __syncthreads();
    if (!(full || (mixed && kflag))) continue;

    v16f sacc[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[s][v] = 0.f;
      const __half* krow = ks + (32 * s + col) * KP + hh * (D / 2);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const v8h kop = *reinterpret_cast<const v8h*>(krow + 8 * c);
        sacc[s] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kop, qop[c], sacc[s], 0, 0, 0);
      }
    }
    const int key0 = j * kBlock;
    float mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = key0 + 32 * s + 8 * (v >> 2) + 4 * hh + (v & 3);
        sacc[s][v] = (key < L) ? sacc[s][v] * c0 : -INFINITY;
        mx = fmaxf(mx, sacc[s][v]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2_hw16(m_run - m_new);
    v8h pop[2][2];
    float psum = 0.f;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float P = exp2_hw16(sacc[s][v] - m_new);
        psum += P;
        pop[s][v >> 3][v & 7] = (_Float16)P;
      }
    l_part = alpha * l_part + psum;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int v = 0; v < 16; ++v) o_acc[ct][v] *= alpha;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const v8h vop = *reinterpret_cast<const v8h*>(&vt[(ct * 32 + col) * VP + 32 * s + 16 * u + 8 * hh]);
          o_acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop, pop[s][u], o_acc[ct], 0, 0, 0);
        }
    }
    m_run = m_new;
  }

  if (!(full || mixed)) return;
  const float l = l_part + __shfl_xor(l_part, 32);
  if (row >= L) return;
  __half* orow = a.out + (long long)b * kp.sb + (long long)h * kp.sh + (long long)row * kp.sl;
  if (full) {
    const float inv_l = 1.0f / l;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = ct * 32 + 8 * g + 4 * hh;
        __half hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = __float2half_rn(o_acc[ct][4 * g + e] * inv_l);
        *reinterpret_cast<uint2*>(orow + ch) = *reinterpret_cast<const uint2*>(hv);
      }
  } else {
    // log-sum-exp merge with the INT4 partial of this row (log2 domain)
    const float m1 = a.part_m[(long long)bh * Lp + row];
    const float l1 = a.part_l[(long long)bh * Lp + row];
    const float mm = fmaxf(m1, m_run);
    const float a1 = (m1 == -INFINITY) ? 0.f : exp2_hw16(m1 - mm);
    const float a2 = (m_run == -INFINITY) ? 0.f : exp2_hw16(m_run - mm);
    const float inv = 1.0f / (a1 * l1 + a2 * l);
    const float* po = a.part_o + ((long long)bh * Lp + row) * D;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = ct * 32 + 8 * g + 4 * hh;
        const float4 p1 = *reinterpret_cast<const float4*>(po + ch);
        const float o1[4] = {p1.x, p1.y, p1.z, p1.w};
        __half hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = __float2half_rn((a1 * o1[e] + a2 * o_acc[ct][4 * g + e]) * inv);
        *reinterpret_cast<uint2*>(orow + ch) = *reinterpret_cast<const uint2*>(hv);
      }
  }
}

hipError_t launch_fp16_attention(const KProblem& kp, const AttnArgs& a, bool whole_call, hipStream_t s) {
  const float c0 = (float)(std::log2(2.718281828459045) / std::sqrt((double)kp.D));
  dim3 grid((kp.L + 127) / 128, kp.H, kp.B);
  if (kp.D == 128)
    hipLaunchKernelGGL((fp16_attn_kernel<128>), grid, dim3(256), 0, s, kp, a, whole_call ? 1 : 0, c0);
  else if (kp.D == 64)
    hipLaunchKernelGGL((fp16_attn_kernel<64>), grid, dim3(256), 0, s, kp, a, whole_call ? 1 : 0, c0);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace rotattn
