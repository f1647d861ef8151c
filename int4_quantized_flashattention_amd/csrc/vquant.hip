// V quantization: per-channel symmetric INT4 over all L tokens of a head,
// the per-64-key-block column sums, and the nibble layout the INT4 attention
// kernel feeds straight into its matrix-core operands.
//
// Method: RotateAttention abstract (arXiv 2607.02584) -- the P.V product of
// the INT4 FlashAttention runs against per-channel INT4 V; the P codes use a
// zero-point of -8, which the column sums of the V codes correct.
//
// Two passes over V because the scale of a channel depends on every token:
//   v_absmax_kernel: per (b, h, 256-token chunk) channel absmax, folded into
//                    a [B][H][D] array with atomicMax on the float bit
//                    patterns (non-negative floats order like their bits);
//   v_quant_kernel:  per (b, h, 64-key block) codes, column sums and the
//                    operand-ordered nibble packing.
#include "common.h"

namespace rotattn {

__global__ void fill_u32_kernel(uint32_t* p, int n, uint32_t val) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = val;
}

template <int D>
__global__ __launch_bounds__(256) void v_absmax_kernel(KProblem kp, const __half* v, uint32_t* absmax_bits) {
  constexpr int G = D / 8;          // 16-byte channel groups per token
  constexpr int RPP = 256 / G;      // token rows per pass
  __shared__ float red[RPP][D + 1];
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, g = t % G, r0 = t / G;
  float m[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = 0.f;
  const __half* base = v + (long long)b * kp.sb + (long long)h * kp.sh + g * 8;
  for (int r = r0; r < 256; r += RPP) {
    const int tok = chunk * 256 + r;
    if (tok >= kp.L) break;
    const uint4 u = *reinterpret_cast<const uint4*>(base + (long long)tok * kp.sl);
    const __half* hv = reinterpret_cast<const __half*>(&u);
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = fmaxf(m[e], fabsf(__half2float(hv[e])));
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[r0][g * 8 + e] = m[e];
  __syncthreads();
  if (t < D) {
    float mx = 0.f;
    for (int r = 0; r < RPP; ++r) mx = fmaxf(mx, red[r][t]);
    atomicMax(&absmax_bits[(b * kp.H + h) * D + t], __float_as_uint(mx));
  }
}

template <int D>
__global__ __launch_bounds__(256) void v_quant_kernel(KProblem kp, const __half* v, const uint32_t* absmax_bits,
                                                      VOut o) {
  constexpr int G = D / 8;
  constexpr int RPP = 256 / G;
  __shared__ float sv[D], rsv[D];
  __shared__ int8_t C[kBlock][D + 4];
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int bh = b * kp.H + h;
  const int t = threadIdx.x;
  if (t < D) {
    const float s = fdiv_rn(__uint_as_float(absmax_bits[bh * D + t]), 7.0f);
    sv[t] = s;
    rsv[t] = (s != 0.f) ? fdiv_rn(1.0f, s) : 0.f;
    if (blk == 0) o.v_scale[bh * D + t] = s;
  }
  __syncthreads();
  const int g = t % G, r0 = t / G;
  const __half* base = v + (long long)b * kp.sb + (long long)h * kp.sh + g * 8;
  float s8[8], rs8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    s8[e] = sv[g * 8 + e];
    rs8[e] = rsv[g * 8 + e];
  }
  for (int r = r0; r < kBlock; r += RPP) {
    const int tok = blk * kBlock + r;
    float c8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) c8[e] = 0.f;
    if (tok < kp.L) {
      const uint4 u = *reinterpret_cast<const uint4*>(base + (long long)tok * kp.sl);
      const __half* hv = reinterpret_cast<const __half*>(&u);
      // code = rne(x / s) as with IEEE division, from x * float(1/s): that
      // product is within 8.93e-7 of the rounded quotient (|x / s| <= 7), so
      // the rounding agrees unless it lies within 1e-6 of a half-integer;
      // there the division is done exactly, behind a wave-uniform branch. No
      // clamp is needed: |x| <= absmax, so both quotients round into [-7, 7].
      float x8[8], q8[8];
      bool near_tie = false;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x8[e] = __half2float(hv[e]);
        q8[e] = fmul_rn(x8[e], rs8[e]);
        c8[e] = rintf(q8[e]);
        near_tie |= s8[e] != 0.f && fabsf(q8[e] - c8[e]) > 0.5f - 1e-6f;
      }
      if (__builtin_amdgcn_ballot_w64(near_tie) != 0ull) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (s8[e] != 0.f && fabsf(q8[e] - c8[e]) > 0.5f - 1e-6f) c8[e] = rintf(fdiv_rn(x8[e], s8[e]));
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) C[r][g * 8 + e] = (int8_t)(int)c8[e];   // a zero scale gives 0 * 0 = 0
  }
  __syncthreads();
  const long long blk_idx = (long long)bh * kp.NB + blk;
  if (t < D) {
    int s = 0;
    for (int r = 0; r < kBlock; ++r) s += C[r][t];
    o.v_colsum[blk_idx * D + t] = s;
  }
  if (t < 2 * D) {
    const int c = t >> 1, hh = t & 1;
    uint32_t w4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {   // q = 2*s + w
      const int s = q >> 1, w = q & 1;
      uint32_t word = 0;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const uint32_t lo = (uint32_t)C[32 * s + 16 * w + 4 * hh + bb][c] & 0xFu;
        const uint32_t hi = (uint32_t)C[32 * s + 16 * w + 8 + 4 * hh + bb][c] & 0xFu;
        word |= (lo | (hi << 4)) << (8 * bb);
      }
      w4[q] = word;
    }
    uint8_t* dst = o.v_codes + (blk_idx * D + c) * 32 + 16 * hh;
    *reinterpret_cast<uint4*>(dst) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  }
}

hipError_t launch_vquant(const KProblem& kp, const __half* v, uint32_t* absmax_bits, const VOut& o, hipStream_t s) {
  const int n = kp.B * kp.H * kp.D;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, absmax_bits, n, 0u);
  dim3 g1((kp.L + 255) / 256, kp.H, kp.B), g2(kp.NB, kp.H, kp.B);
  if (kp.D == 128) {
    hipLaunchKernelGGL((v_absmax_kernel<128>), g1, dim3(256), 0, s, kp, v, absmax_bits);
    hipLaunchKernelGGL((v_quant_kernel<128>), g2, dim3(256), 0, s, kp, v, absmax_bits, o);
  } else if (kp.D == 64) {
    hipLaunchKernelGGL((v_absmax_kernel<64>), g1, dim3(256), 0, s, kp, v, absmax_bits);
    hipLaunchKernelGGL((v_quant_kernel<64>), g2, dim3(256), 0, s, kp, v, absmax_bits, o);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rotattn
