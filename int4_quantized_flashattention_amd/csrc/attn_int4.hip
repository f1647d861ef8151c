// Fused INT4 flash-attention loop on the gfx950 matrix cores.
//
// Method: RotateAttention abstract (arXiv 2607.02584) -- mixed-precision INT4
// FlashAttention with integer Q.K^T, the range-optimized P quantization
// (fixed scale 1/15, zero-point -8) and integer P.V against per-channel INT4
// V; loop structure and recurrences from RainFusion2.0, section 3.1
// "Blockwise Sparse" (m <- max(m, rowmax S); P = exp(S - m);
// l <- exp(m_old - m) l + rowsum P; O <- diag(exp(m_old - m)) O + P V;
// O / l at the end), in the log2 domain, over key blocks of 64 in ascending
// order; tiles routed to the FP16 path are skipped like masked blocks.
//
// Layout of the work (one workgroup = 4 waves = 128 query rows of one head):
//  * S^T = K Q^T with v_mfma_i32_32x32x32_i8: K codes are the A operand (rows
//    = keys), Q codes the B operand (columns = queries). Each lane then owns
//    one query column and 16 of the 32 keys of a 32 x 32 tile, so the row
//    max and row sum are in-lane plus one exchange with lane ^ 32, and the P
//    codes are already laid out as the B operand of the next product.
//  * O^T = V^T P^T with the same instruction: V codes (A, rows = channels,
//    stored by the V quantizer in exactly this operand order) times the P
//    codes (B). The zero-point correction is applied inside the product: the
//    kernel feeds the shifted code pq + 8 = rne(15 P) in [0, 15], and
//    sum (pq + 8) v = sum pq v + 8 colsum(v) exactly (integer identity).
//  * INT4 nibbles become int8 operands with two ANDs and a shift per 8 codes
//    (each value times 16; the factors 256 and 16 are folded into the float
//    scales exactly).
//  * K and V tiles of the current key block are staged through LDS once per
//    workgroup.
#include "common.h"

#include <climits>

namespace rotattn {

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

template <int DP, int DV, bool DUMP>
__global__ __launch_bounds__(256) void int4_attn_kernel(KProblem kp, AttnArgs a, float c0) {
  constexpr int NC = DP / 32;            // 32-deep slices of the rotated head dim
  constexpr int NCT = DV / 32;           // 32-channel output tiles
  constexpr int KT_BYTES = kBlock * DP / 2;
  constexpr int VT_BYTES = DV * 32;
  constexpr int QROW = DP / 2;           // code bytes per token
  constexpr int HALF = DP / 4;           // code bytes of one lane half
  __shared__ __attribute__((aligned(16))) uint8_t ks[KT_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t vs[VT_BYTES];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int L = kp.L, Lp = kp.Lp, NB = kp.NB;

  int b, h, row_base, unit_idx = 0;
  if (DUMP) {
    unit_idx = blockIdx.x;
    const int u = a.units[unit_idx];
    if (u < 0 || u >= kp.B * kp.H * NB) return;   // unit out of range: nothing to dump
    const int qb = u % NB, bh0 = u / NB;
    b = bh0 / kp.H;
    h = bh0 - b * kp.H;
    row_base = qb * kBlock;
  } else {
    b = blockIdx.z;
    h = blockIdx.y;
    row_base = blockIdx.x * 128;
  }
  const int bh = b * kp.H + h;
  const int wrow = row_base + 32 * wave;
  const bool active = (wrow < L) && (!DUMP || wave < 2);
  const int qblk = wrow / kBlock;
  bool fp16_row = false;
  if (active) {
    fp16_row = (a.head_mask != nullptr && a.head_mask[bh] != 0) || (a.route && a.q_flag[bh * NB + qblk] != 0);
  }
  const bool work = active && !fp16_row;
  const bool mixed = work && a.route && a.head_kflag[bh] != 0;
  if (!__syncthreads_or(work)) return;

  // Q codes of this lane's query (column) and half of the rotated dims.
  v4i qop[NC];
  float cq = 0.f;
  if (work) {
    const uint8_t* qrow = a.q_codes + ((long long)bh * Lp + wrow + col) * QROW + hh * HALF;
#pragma unroll
    for (int c = 0; c < NC; ++c) qop[c] = unpack16(*reinterpret_cast<const uint2*>(qrow + 8 * c));
    cq = fmul_rn(a.q_scale[bh * NB + qblk], c0);
  }

  float m_run = -INFINITY;
  float l_part = 0.f;
  v16f o_acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int v = 0; v < 16; ++v) o_acc[ct][v] = 0.f;

  const uint8_t* kbase_g = a.k_codes + (long long)bh * Lp * QROW;
  const uint8_t* vbase_g = a.v_codes + (long long)bh * NB * VT_BYTES;

  for (int j = 0; j < NB; ++j) {
    if (a.route && a.k_flag[bh * NB + j] != 0) continue;   // FP16 tile: the other path takes it
    __syncthreads();
    {
      const uint8_t* kt = kbase_g + (long long)j * KT_BYTES;
      for (int o = threadIdx.x * 16; o < KT_BYTES; o += 256 * 16)
        *reinterpret_cast<uint4*>(ks + o) = *reinterpret_cast<const uint4*>(kt + o);
      const uint8_t* vt = vbase_g + (long long)j * VT_BYTES;
      for (int o = threadIdx.x * 16; o < VT_BYTES; o += 256 * 16)
        *reinterpret_cast<uint4*>(vs + o) = *reinterpret_cast<const uint4*>(vt + o);
    }
    __syncthreads();
    if (!work) continue;

    // S^T tile (times 256): two 32-key halves of the block.
    v16i sacc[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[s][v] = 0;
      const uint8_t* krow = ks + (32 * s + col) * QROW + hh * HALF;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const v4i kop = unpack16(*reinterpret_cast<const uint2*>(krow + 8 * c));
        sacc[s] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop, qop[c], sacc[s], 0, 0, 0);
      }
    }
    // c = float(float(sq c0) sk); the operands carry a factor 256, folded in exactly.
    const float ct_scale = fmul_rn(fmul_rn(cq, a.k_scale[bh * NB + j]), 1.0f / 256.0f);
    const int key0 = j * kBlock;
    int mx = INT_MIN;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = key0 + 32 * s + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (key < L) mx = max(mx, sacc[s][v]);
      }
    mx = max(mx, __shfl_xor(mx, 32));
    // max over the block of float(acc) * c = float(max acc) * c, as c >= 0
    const float m_blk = fmul_rn((float)mx, ct_scale);
    const float m_new = fmaxf(m_run, m_blk);
    const float alpha = exp2_hw(fsub_rn(m_run, m_new));

    v4i pop[2];
    float psum = 0.f;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        uint32_t word = 0;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int v = 4 * kq + bb;
          const int key = key0 + 32 * s + 8 * kq + 4 * hh + bb;
          float P = 0.f;
          if (key < L) P = exp2_hw(fsub_rn(fmul_rn((float)sacc[s][v], ct_scale), m_new));
          psum += P;
          const uint32_t code = (uint32_t)(int)rintf(fmul_rn(15.0f, P));   // pq + 8 in [0, 15]
          word |= code << (8 * bb);
          if (DUMP) {
            const int r = 32 * wave + col;
            if (wrow + col < L) {
              const long long di = ((long long)unit_idx * kBlock + r) * Lp + key;
              a.d_acc[di] = sacc[s][v] >> 8;
              a.d_pq[di] = (int8_t)((int)code - 8);
            }
          }
        }
        pop[s][kq] = (int)word;
      }
    l_part = alpha * l_part + psum;

#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      v16i pacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) pacc[v] = 0;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint8_t* vrow = vs + (ct * 32 + col) * 32 + 16 * hh + 8 * s;
        const v4i vop = unpack16(*reinterpret_cast<const uint2*>(vrow));
        pacc = __builtin_amdgcn_mfma_i32_32x32x32_i8(vop, pop[s], pacc, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) o_acc[ct][v] = alpha * o_acc[ct][v] + (float)pacc[v];
      if (DUMP) {
        const int r = 32 * wave + col;
        if (wrow + col < L) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int ch = ct * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
            a.d_pv[(((long long)unit_idx * kBlock + r) * NB + j) * DV + ch] = pacc[v] >> 4;
          }
        }
      }
    }
    m_run = m_new;
    if (DUMP && hh == 0 && wrow + col < L)
      a.d_m[((long long)unit_idx * kBlock + 32 * wave + col) * NB + j] = m_run;
  }

  if (DUMP || !work) return;
  const float l = l_part + __shfl_xor(l_part, 32);
  const int row = wrow + col;
  if (row >= L) return;
  const float* svp = a.v_scale + (long long)bh * DV;
  if (!mixed) {
    const float inv_l = 1.0f / l;
    __half* orow = a.out + (long long)b * kp.sb + (long long)h * kp.sh + (long long)row * kp.sl;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = ct * 32 + 8 * g + 4 * hh;
        __half hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          hv[e] = __float2half_rn(o_acc[ct][4 * g + e] * (svp[ch + e] * (1.0f / 240.0f)) * inv_l);
        *reinterpret_cast<uint2*>(orow + ch) = *reinterpret_cast<const uint2*>(hv);
      }
  } else {
    float* po = a.part_o + ((long long)bh * Lp + row) * DV;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = ct * 32 + 8 * g + 4 * hh;
        float4 f;
        f.x = o_acc[ct][4 * g + 0] * (svp[ch + 0] * (1.0f / 240.0f));
        f.y = o_acc[ct][4 * g + 1] * (svp[ch + 1] * (1.0f / 240.0f));
        f.z = o_acc[ct][4 * g + 2] * (svp[ch + 2] * (1.0f / 240.0f));
        f.w = o_acc[ct][4 * g + 3] * (svp[ch + 3] * (1.0f / 240.0f));
        *reinterpret_cast<float4*>(po + ch) = f;
      }
    if (hh == 0) {
      a.part_m[(long long)bh * Lp + row] = m_run;
      a.part_l[(long long)bh * Lp + row] = l;
    }
  }
}

template <int DP, int DV>
static hipError_t launch_int4_t(const KProblem& kp, const AttnArgs& a, bool dump, float c0, hipStream_t s) {
  if (dump) {
    hipLaunchKernelGGL((int4_attn_kernel<DP, DV, true>), dim3(a.n_units), dim3(256), 0, s, kp, a, c0);
  } else {
    dim3 grid((kp.L + 127) / 128, kp.H, kp.B);
    hipLaunchKernelGGL((int4_attn_kernel<DP, DV, false>), grid, dim3(256), 0, s, kp, a, c0);
  }
  return hipGetLastError();
}

hipError_t launch_int4_attention(const KProblem& kp, const AttnArgs& a, bool dump, hipStream_t s) {
  const float c0 = (float)(std::log2(2.718281828459045) / std::sqrt((double)kp.D));
  if (kp.Dp == 128 && kp.D == 128) return launch_int4_t<128, 128>(kp, a, dump, c0, s);
  if (kp.Dp == 192 && kp.D == 128) return launch_int4_t<192, 128>(kp, a, dump, c0, s);
  if (kp.Dp == 64 && kp.D == 64) return launch_int4_t<64, 64>(kp, a, dump, c0, s);
  if (kp.Dp == 192 && kp.D == 64) return launch_int4_t<192, 64>(kp, a, dump, c0, s);
  return hipErrorInvalidValue;
}

}  // namespace rotattn
