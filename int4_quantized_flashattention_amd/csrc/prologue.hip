// Q/K prologue: 3D RoPE -> RoPE-aware rotation -> per-64-token INT4
// quantization with nibble-packed stores and the block error flag; optionally
// the RoPE'd copies for the FP16 path and the block sums for block sparsity.
//
// Method: RotateAttention abstract (arXiv 2607.02584) -- 3D RoPE on Q and K,
// a RoPE-aware orthonormal rotation (the online Walsh-Hadamard after RoPE, over
// the head dim or per RoPE group, or the mergeable per-pair rotation folded
// into RoPE's angles), symmetric INT4 quantization, and selective FP16
// fallback for blocks whose quantization error is too large. Block sums:
// RainFusion2.0, section 3.2 (block means as representative tokens).
//
// One workgroup of 256 threads handles one 64-token block of one (b, h,
// tensor). The block is read once (16-byte loads; 4-byte pairs in the
// per-group register kernel), rotated in registers (and LDS where the layout
// needs it), and written once as nibble-packed codes: HBM traffic is the
// compulsory 2 bytes in / D'/2 bytes out per token and head dim. Three
// kernels: the register kernel (even RoPE groups, full or pair rotation; a
// second instance also writes the copies and block sums), the per-group
// register kernel (even groups, no copies or sums), and the LDS-tile kernel
// for everything else.
//
// Floating-point contract (both sides of the parity tests follow it): each
// RoPE product and sum is rounded separately (no FMA; the library is built
// with -ffp-contract=off and uses __fmul_rn and friends), the Hadamard
// butterflies run in stage order h = 1, 2, 4, ..., then one multiply by
// float(1/sqrt(n)); scale = absmax / 7 and code = rne(x / scale) as with
// IEEE division (x * float(1/scale), divided exactly near rounding ties). The
// error-to-signal sums of the block flag use fused multiply-adds in float32
// (the flag is exact except where that ratio lies next to the threshold).
#include "common.h"

namespace rotattn {

// cos/sin of every (axis, position, pair): angle = pos * base^(-2i / g_rot)
// + phase (phase: the mergeable rotation folded into RoPE, else 0), evaluated
// in double and rounded once to float. Also zeroes a small u32 array (the
// per-head flag summary) so that one launch prepares both.
__global__ void rope_table_kernel(KProblem kp, float* tab, uint32_t* zero_u32, int n_zero, double phase) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (zero_u32 != nullptr && i < n_zero) zero_u32[i] = 0u;
  int rem = i;
  for (int a = 0; a < 3; ++a) {
    const int npos = (a == 0) ? kp.T : (a == 1) ? kp.Hh : kp.W;
    const int np = kp.npair[a];
    const int n = npos * np;
    if (rem < n) {
      const int p = rem / np, pi = rem - (rem / np) * np;
      const double th = pow(kp.base, -(2.0 * pi) / (double)(2 * np));
      const double ang = (double)p * th + phase;
      tab[kp.tab_off[a] + rem] = (float)cos(ang);
      tab[kp.tab_off[a] + n + rem] = (float)sin(ang);
      return;
    }
    rem -= n;
  }
}

template <int D>
__device__ __forceinline__ void load_block_to_lds(const KProblem& kp, const __half* x, int b, int h, int blk,
                                                  float (*Y)[D + 4]) {
  constexpr int PER = D / 4;  // halves per thread (4 threads per token)
  const int t = threadIdx.x;
  const int tok = t >> 2, part = t & 3;
  const int tg = blk * kBlock + tok;
  float vals[PER];
  if (tg < kp.L) {
    const __half* src = x + (long long)b * kp.sb + (long long)h * kp.sh + (long long)tg * kp.sl + part * PER;
#pragma unroll
    for (int c = 0; c < PER / 8; ++c) {
      uint4 u = reinterpret_cast<const uint4*>(src)[c];
      const __half* hv = reinterpret_cast<const __half*>(&u);
#pragma unroll
      for (int e = 0; e < 8; ++e) vals[c * 8 + e] = __half2float(hv[e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) vals[e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) Y[tok][part * PER + e] = vals[e];
}

// RoPE in place on the LDS tile (call after the tile's loads, with the whole
// workgroup; it synchronizes before reading the tile and the caller
// synchronizes after it). Thread t owns pair t % 64 (of the npair[0] +
// npair[1] + npair[2] pairs) for the tokens t / 64 + 4 i; the video
// coordinates of the block's tokens are computed once into `coord`. With PAIR the
// mergeable rotation is folded in: the tables carry the extra angle and the
// pairs of text tokens turn by it alone.
template <int D, bool PAIR = false>
__device__ __forceinline__ void rope_lds(const KProblem& kp, const float* tab, int blk, float (*Y)[D + 4],
                                         int (*coord)[3]) {
  const int tid = threadIdx.x;
  {
    __syncthreads();   // the tile is loaded; coord may be rewritten
    if (tid < kBlock) {
      const int idx = blk * kBlock + tid - kp.prefix;
      const int hw = kp.Hh * kp.W;
      const int t = idx >= 0 && hw > 0 ? idx / hw : 0;
      const int rem = idx >= 0 && hw > 0 ? idx - t * hw : 0;
      const int hq = kp.W > 0 ? rem / kp.W : 0;
      coord[tid][0] = t;
      coord[tid][1] = hq;
      coord[tid][2] = rem - hq * kp.W;
    }
    __syncthreads();
  }
  const int npt = kp.npair[0] + kp.npair[1] + kp.npair[2];
  int pr = tid & 63;
  if (pr >= npt) return;   // D = 64: 31 pairs
  int a = 0;
  if (pr >= kp.npair[0]) { pr -= kp.npair[0]; a = 1; }
  if (a == 1 && pr >= kp.npair[1]) { pr -= kp.npair[1]; a = 2; }
  const int d0 = kp.off[a] + 2 * pr;
  const int npos = (a == 0) ? kp.T : (a == 1) ? kp.Hh : kp.W;
  const float* ctab = tab + kp.tab_off[a] + pr;
  const float* stab = ctab + npos * kp.npair[a];
  const int stride = kp.npair[a];
  // this thread's 16 tokens: every table load first (one memory latency, not
  // sixteen), then the rotations; tokens past L and text tokens read
  // position 0 and are left alone (text tokens turn by the pair angle alone
  // with PAIR)
  constexpr int NT = kBlock / 4;
  float cv[NT], sv[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int tok = (tid >> 6) + 4 * i;
    const int tg = blk * kBlock + tok;
    const int pos = (tg < kp.L && tg >= kp.prefix) ? coord[tok][a] : 0;
    cv[i] = ctab[pos * stride];
    sv[i] = stab[pos * stride];
  }
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int tok = (tid >> 6) + 4 * i;
    const int tg = blk * kBlock + tok;
    if (tg >= kp.L) break;
    float c = cv[i], s = sv[i];
    if (tg < kp.prefix) {
      if (!PAIR) continue;
      c = kp.pair_c;
      s = kp.pair_s;
    }
    const float x0 = Y[tok][d0], x1 = Y[tok][d0 + 1];
    Y[tok][d0] = fsub_rn(fmul_rn(x0, c), fmul_rn(x1, s));
    Y[tok][d0 + 1] = fadd_rn(fmul_rn(x0, s), fmul_rn(x1, c));
  }
}

template <int D>
__device__ __forceinline__ void store_rope_copy(const KProblem& kp, int b, int h, int blk, float (*Y)[D + 4],
                                                __half* dst) {
  constexpr int PER = D / 4;
  const int t = threadIdx.x;
  const int tok = t >> 2, part = t & 3;
  const int tg = blk * kBlock + tok;
  if (tg >= kp.L) return;
  __half* d = dst + ((long long)(b * kp.H + h) * kp.L + tg) * D + part * PER;
#pragma unroll
  for (int c = 0; c < PER / 8; ++c) {
    uint4 u;
    __half* hv = reinterpret_cast<__half*>(&u);
#pragma unroll
    for (int e = 0; e < 8; ++e) hv[e] = __float2half_rn(Y[tok][part * PER + c * 8 + e]);
    reinterpret_cast<uint4*>(d)[c] = u;
  }
}

// floor(n / d) for 0 <= n < 2^22 and 1 <= d <= 2^22: float(n) rcp(d) has a
// relative error of at most 1.5 ulp, so it is within 3/4 of n / d and its
// truncation is off by at most one either way; one step each way corrects it
// (the products fit the 24-bit multiplier)
__device__ __forceinline__ int quot_small(int n, int d) {
  int t = (int)((float)n * __builtin_amdgcn_rcpf((float)d));
  t -= (__mul24(t, d) > n) ? 1 : 0;
  t += (__mul24(t + 1, d) <= n) ? 1 : 0;
  return t;
}

// Sum over the valid tokens of a 64-token block, per dim, of the chunks that
// the threads of the register kernel hold (thread 64 w + l: token
// 16 w + l / PARTS, chunk l % PARTS, zero past L): within a wave the lanes
// PARTS apart are summed by DPP row rotations (by PARTS up to 8 within each row
// of 16) and the permlane swaps of rows 16 and 32 apart; the four wave sums meet
// in LDS. Written to dst[0, D) by the first D threads. Called by the whole
// workgroup.
template <int D>
__device__ __forceinline__ void block_sum_chunks(const float (&v)[32], float* dst, float* bs) {
  constexpr int PARTS = D / 32;
  float sm[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) sm[e] = v[e];
  auto row_ror_add = [&](auto ctl_tag) __attribute__((always_inline)) {
    constexpr int kCtl = decltype(ctl_tag)::value;   // DPP row_ror:n = 0x120 + n
#pragma unroll
    for (int e = 0; e < 32; ++e)
      sm[e] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sm[e]), kCtl, 0xF, 0xF, false));
  };
  if constexpr (PARTS == 2) row_ror_add(std::integral_constant<int, 0x122>());
  row_ror_add(std::integral_constant<int, 0x124>());
  row_ror_add(std::integral_constant<int, 0x128>());
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const auto w16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(sm[e]), __float_as_uint(sm[e]), false, false);
    sm[e] = __uint_as_float(w16[0]) + __uint_as_float(w16[1]);   // this lane's value and lane ^ 16's
    const auto w32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sm[e]), __float_as_uint(sm[e]), false, false);
    sm[e] = __uint_as_float(w32[0]) + __uint_as_float(w32[1]);   // and lane ^ 32's
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane < PARTS) {
#pragma unroll
    for (int e = 0; e < 32; ++e) bs[wave * D + 32 * lane + e] = sm[e];
  }
  __syncthreads();
  const int d = threadIdx.x;
  if (d < D) dst[d] = (bs[d] + bs[D + d]) + (bs[2 * D + d] + bs[3 * D + d]);
}

// v of lane ^ MASK (MASK 1 or 2) within the lane's aligned group of four, by
// a DPP quad permutation (no LDS round trip). The 32-value chunks of one
// token sit in consecutive lanes from a multiple of PARTS (4, or 2 and 6 with
// MASK 1 only), so the Hadamard partners of stages 32 and 64 are such lanes.
template <int MASK>
__device__ __forceinline__ float quad_xor(float v) {
  constexpr int kQuadPerm = MASK == 1 ? 0xB1 : 0x4E;   // [1,0,3,2] : [2,3,0,1]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kQuadPerm, 0xF, 0xF, true));
}

__device__ __forceinline__ float block_reduce_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_reduce_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Shape of the prologue's work: each token's rotated row (D' values) in
// 32-value chunks, one chunk per task, one task per thread and round.
template <int D, int ROT>
struct ProShape {
  static constexpr int DP = (ROT == 1) ? 192 : D;
  static constexpr int N = (ROT == 1) ? 64 : D;       // Walsh-Hadamard size (ROT 2: no Hadamard)
  static constexpr int PARTS = DP / 32;               // 32-value chunks per token
  static constexpr int TASKS = kBlock * PARTS;        // multiple of 64
  static constexpr int ROUNDS = (TASKS + 255) / 256;
};

// Rotation, quantization and stores of one 64-token block, given the RoPE'd
// values of each task's chunk in v (task = threadIdx.x + 256 r = token * PARTS
// + chunk): the Walsh-Hadamard on 32-value chunks (stages 1..16 in registers,
// 32 and 64 across lanes), the block scale, the codes, the scale and the error
// flag. Called by the whole workgroup.
template <int D, int ROT>
__device__ __forceinline__ void rotate_quantize(const KProblem& kp, const QKOut& o, int b, int h, int blk,
                                                int tensor, float (&v)[ProShape<D, ROT>::ROUNDS][32], float* red) {
  using S = ProShape<D, ROT>;
  constexpr int DP = S::DP, N = S::N, PARTS = S::PARTS, TASKS = S::TASKS, ROUNDS = S::ROUNDS;
  float amax = 0.f;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int task = threadIdx.x + 256 * r;
    if (task < TASKS) {  // wave-uniform
      const int part = task - (task / PARTS) * PARTS;
      if constexpr (ROT != 2) {
#pragma unroll
      for (int hs = 1; hs < 32; hs <<= 1) {
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          if ((j & hs) == 0) {
            const float a0 = v[r][j], b0 = v[r][j + hs];
            v[r][j] = fadd_rn(a0, b0);
            v[r][j + hs] = fsub_rn(a0, b0);
          }
        }
      }
#pragma unroll
      for (int hs = 32; hs < N; hs <<= 1) {
        const int mask = hs >> 5;
        const bool upper = (part & mask) != 0;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const float other = mask == 1 ? quad_xor<1>(v[r][j]) : quad_xor<2>(v[r][j]);
          v[r][j] = upper ? fsub_rn(other, v[r][j]) : fadd_rn(v[r][j], other);
        }
      }
      const float rn = (N == 128) ? 0.08838834764831845f : (N == 64) ? 0.125f : 0.f;
#pragma unroll
      for (int j = 0; j < 32; ++j) v[r][j] = fmul_rn(v[r][j], rn);
      }   // ROT != 2
#pragma unroll
      for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[r][j]));
    }
  }
  amax = block_reduce_max(amax, red);
  const float s = fdiv_rn(amax, 7.0f);
  const float rs = (s != 0.f) ? fdiv_rn(1.0f, s) : 0.f;

  float se = 0.f, sx = 0.f;
  uint8_t* codes = tensor ? o.k_codes : o.q_codes;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int task = threadIdx.x + 256 * r;
    if (task < TASKS) {
      const int tok = task / PARTS, part = task - (task / PARTS) * PARTS;
      uint32_t words[4] = {0u, 0u, 0u, 0u};
      // rne(x / s) with IEEE division: x * float(1/s) is within 8.4e-7 of
      // x / s (|x / s| <= 7), so away from the half-integers the rounding
      // agrees; within 1e-6 of one the division is done exactly. The
      // divisions sit behind a wave-uniform branch taken only when some lane
      // of the wave has such a value (otherwise the compiler evaluates them
      // for every element and selects).
      // A value is near a half-integer when it is more than 0.5 - 1e-6 from
      // its nearest integer (qd - rint(qd) is exact). No clamp to [-7, 7] is
      // needed: |x| <= amax, so |x * float(1/s)| <= 7 (1 + 3 2^-24) < 7.5 and
      // the exact quotient is at most 7.
      float qd[32], cq[32];
      bool near_tie = false;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        qd[j] = fmul_rn(v[r][j], rs);
        cq[j] = rintf(qd[j]);
        near_tie |= fabsf(qd[j] - cq[j]) > 0.5f - 1e-6f;
      }
      if (__builtin_amdgcn_ballot_w64(near_tie && s != 0.f) != 0ull) {
#pragma unroll
        for (int j = 0; j < 32; ++j)
          if (s != 0.f && fabsf(qd[j] - cq[j]) > 0.5f - 1e-6f) cq[j] = rintf(fdiv_rn(v[r][j], s));
      }
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        // (s = 0 only for an all-zero block, whose codes are 0 already)
        const float c = cq[j];
        // the error and energy sums with fused multiply-adds: the residual
        // v - s c is exact, the sums are rounded once per term
        const float e = __builtin_fmaf(-s, c, v[r][j]);
        se = __builtin_fmaf(e, e, se);
        sx = __builtin_fmaf(v[r][j], v[r][j], sx);
        const uint32_t nib = (uint32_t)((int)c) & 0xFu;
        words[j >> 3] |= nib << (4 * (j & 7));
      }
      const int tg = blk * kBlock + tok;
      uint8_t* dst = codes + ((long long)(b * kp.H + h) * kp.Lp + tg) * (DP / 2) + 16 * part;
      *reinterpret_cast<uint4*>(dst) = make_uint4(words[0], words[1], words[2], words[3]);
    }
  }
  se = block_reduce_sum(se, red);
  sx = block_reduce_sum(sx, red);
  if (threadIdx.x == 0) {
    const long long bi = (long long)(b * kp.H + h) * kp.NB + blk;
    (tensor ? o.k_scale : o.q_scale)[bi] = s;
    const float nsr = (sx > 0.f) ? se / sx : 0.f;
    const uint8_t flag = (nsr > kp.tau) ? 1 : 0;
    (tensor ? o.k_flag : o.q_flag)[bi] = flag;
    if (tensor == 1 && flag) atomicAdd(&o.head_kflag[b * kp.H + h], 1u);   // flagged K blocks of the head
  }
}


// Grid (NB, H, 2B): blockIdx.z = 2*b + tensor (0 = Q, 1 = K). The block is
// staged in LDS (RoPE thread per pair, rotation thread per chunk); this
// kernel also writes the RoPE'd copies and the block sums when asked.
template <int D, int ROT>
__global__ __launch_bounds__(256) void qk_prologue_kernel(KProblem kp, const __half* q, const __half* k,
                                                          const float* tab, QKOut o) {
  using S = ProShape<D, ROT>;
  constexpr int PARTS = S::PARTS, TASKS = S::TASKS, ROUNDS = S::ROUNDS;
  __shared__ float Y[kBlock][D + 4];
  __shared__ float red[4];
  __shared__ int coord[kBlock][3];

  const int blk = blockIdx.x, h = blockIdx.y;
  const int b = blockIdx.z >> 1, tensor = blockIdx.z & 1;
  const __half* x = tensor ? k : q;

  load_block_to_lds<D>(kp, x, b, h, blk, Y);
  rope_lds<D, ROT == 2>(kp, tab, blk, Y, coord);
  __syncthreads();
  __half* rcopy = tensor ? o.k_rope : o.q_rope;
  if (rcopy != nullptr) store_rope_copy<D>(kp, b, h, blk, Y, rcopy);
  // block sum of the RoPE'd rows over the valid tokens (ascending order), the
  // representative token of block-sparse attention before its division by the
  // count (RainFusion2.0, section 3.2)
  float* bsum = tensor ? o.k_bsum : o.q_bsum;
  if (bsum != nullptr) {
    const int n = min(kBlock, kp.L - blk * kBlock);
    float* dst = bsum + ((long long)(b * kp.H + h) * kp.NB + blk) * D;
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
      float acc = 0.f;
      for (int t = 0; t < n; ++t) acc = fadd_rn(acc, Y[t][d]);
      dst[d] = acc;
    }
  }

  float v[ROUNDS][32];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int task = threadIdx.x + 256 * r;
    if (task < TASKS) {  // wave-uniform
      const int tok = task / PARTS, part = task - (task / PARTS) * PARTS;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int p = 32 * part + e;
        if (ROT == 1) {
          const int g = p >> 6, oo = p & 63;
          v[r][e] = (oo < kp.split[g]) ? Y[tok][kp.off[g] + oo] : 0.f;
        } else {
          v[r][e] = Y[tok][p];
        }
      }
    }
  }
  rotate_quantize<D, ROT>(kp, o, b, h, blk, tensor, v, red);
}

// The same without the LDS tile, when every RoPE group starts at an even dim
// and has an even size, so that each pair (2i, 2i + 1) lies inside one
// 32-value chunk: each thread loads its chunk of one token with 16-byte loads
// and applies RoPE in registers (the same products and sums, rounded the same
// way), then the rotation and quantization as above. No LDS beyond the
// reductions, so the occupancy is set by the registers. ROT 0 (full Hadamard)
// or 2 (pair rotation folded into RoPE). EXTRA: the instance that may also
// write the RoPE'd copies and the block sums (more registers; the common call
// asks for neither).
template <int D, int ROT, bool EXTRA>
__global__ __launch_bounds__(256) void qk_prologue_reg_kernel(KProblem kp, const __half* q, const __half* k,
                                                              const float* tab, QKOut o) {
  static_assert(ROT == 0 || ROT == 2, "chunks of the unpadded row");
  using S = ProShape<D, ROT>;
  constexpr int PARTS = S::PARTS, TASKS = S::TASKS;
  static_assert(S::ROUNDS == 1, "one chunk per thread");
  __shared__ float red[4];
  __shared__ float bs[EXTRA ? 4 * D : 1];   // block sums: one partial row per wave
  const int blk = blockIdx.x, h = blockIdx.y;
  const int b = blockIdx.z >> 1, tensor = blockIdx.z & 1;
  const __half* x = tensor ? k : q;

  float v[1][32];
#pragma unroll
  for (int e = 0; e < 32; ++e) v[0][e] = 0.f;
  const int task = threadIdx.x;
  if (task < TASKS) {  // wave-uniform
    const int tok = task / PARTS, part = task - tok * PARTS;
    const int tg = blk * kBlock + tok;
    if (tg < kp.L) {
      const __half* src = x + (long long)b * kp.sb + (long long)h * kp.sh + (long long)tg * kp.sl + 32 * part;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 u = reinterpret_cast<const uint4*>(src)[c];
        const __half* hv = reinterpret_cast<const __half*>(&u);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[0][8 * c + e] = __half2float(hv[e]);
      }
      // grid coordinates of the token (text tokens: none)
      const bool text = tg < kp.prefix;
      int coord[3] = {0, 0, 0};
      if (!text) {
        const int idx = tg - kp.prefix, hw = kp.Hh * kp.W;
        int t, hq;
        if (kp.L <= (1 << 22)) {   // uniform
          t = quot_small(idx, hw);
          hq = quot_small(idx - t * hw, kp.W);
        } else {
          t = idx / hw;
          hq = (idx - t * hw) / kp.W;
        }
        coord[0] = t;
        coord[1] = hq;
        coord[2] = idx - t * hw - hq * kp.W;
      }
      // cos/sin of the chunk's 16 pairs, every table load first (video tokens
      // only: the tables have no entries for text tokens, and with no video
      // tokens at all none). Pair p = 16 part + i of the row (dims 2p, 2p + 1)
      // lies in axis a = [p >= off[1]/2] + [p >= off[2]/2] at index
      // p - off[a]/2 of that axis; its cos is table float
      // tab_off[a] + pos_a npair[a] + p - off[a]/2 and its sin npos_a npair[a]
      // floats further. Per lane and axis that is a byte offset oc[a] (os[a])
      // plus 4 i; the loads add it to the table base in scalar registers.
      // oc[a] >= 0: with even groups off[a]/2 = sum of npair over the axes
      // before a, and tab_off[a] = sum of 2 npos npair over them, npos >= 1.
      float cv[16], sv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        cv[i] = 1.f;
        sv[i] = 0.f;
      }
      if (!text) {
        const int p0 = 16 * part;
        uint32_t oc[3], os[3];
#pragma unroll
        for (int a = 0; a < 3; ++a) {
          const int npos = a == 0 ? kp.T : a == 1 ? kp.Hh : kp.W;
          oc[a] = 4u * (uint32_t)max(kp.tab_off[a] + coord[a] * kp.npair[a] - (kp.off[a] >> 1) + p0, 0);
          os[a] = oc[a] + 4u * (uint32_t)(npos * kp.npair[a]);
        }
        const int t1 = (kp.off[1] >> 1) - p0, t2 = (kp.off[2] >> 1) - p0;   // first i in axis 1, axis 2
        const char* tb = reinterpret_cast<const char*>(tab);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const bool ge1 = i >= t1, ge2 = i >= t2;
          const uint32_t co = (ge2 ? oc[2] : ge1 ? oc[1] : oc[0]) + 4u * i;
          const uint32_t so = (ge2 ? os[2] : ge1 ? os[1] : os[0]) + 4u * i;
          cv[i] = *reinterpret_cast<const float*>(tb + co);
          sv[i] = *reinterpret_cast<const float*>(tb + so);
        }
      }
      if (!text || ROT == 2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float c = text ? kp.pair_c : cv[i], s = text ? kp.pair_s : sv[i];
          const float x0 = v[0][2 * i], x1 = v[0][2 * i + 1];
          v[0][2 * i] = fsub_rn(fmul_rn(x0, c), fmul_rn(x1, s));
          v[0][2 * i + 1] = fadd_rn(fmul_rn(x0, s), fmul_rn(x1, c));
        }
      }
      // the RoPE'd fp16 copy of the chunk (the FP16 path's input)
      __half* rcopy = tensor ? o.k_rope : o.q_rope;
      if (EXTRA && rcopy != nullptr) {
        __half* dst = rcopy + ((long long)(b * kp.H + h) * kp.L + tg) * D + 32 * part;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint4 u;
          __half* hv = reinterpret_cast<__half*>(&u);
#pragma unroll
          for (int e = 0; e < 8; ++e) hv[e] = __float2half_rn(v[0][8 * c + e]);
          reinterpret_cast<uint4*>(dst)[c] = u;
        }
      }
    }
  }
  // block sum of the RoPE'd rows over the valid tokens, the representative
  // token of block-sparse attention before its division by the count
  // (RainFusion2.0, section 3.2)
  float* bsum = tensor ? o.k_bsum : o.q_bsum;
  if (EXTRA && bsum != nullptr) block_sum_chunks<D>(v[0], bsum + ((long long)(b * kp.H + h) * kp.NB + blk) * D, bs);
  rotate_quantize<D, ROT>(kp, o, b, h, blk, tensor, v, red);
}

// The per-group layout (rotation 1: each RoPE group Walsh-Hadamard rotated
// alone, zero-padded to 64) without the LDS tile, for even RoPE groups when
// neither RoPE'd copies nor block sums are asked for (the copies, written a
// pair at a time from here, made the call slower than the LDS tile's 16-byte
// stores). Task (token, chunk c of six) holds dims [32 hf, +32) of group
// g = c / 2 (hf = c % 2), zero past the group's size (the padding), loaded and
// RoPE'd a pair at a time in registers; two rounds of 256 tasks, then the
// rotation and quantization as above.
template <int D>
__global__ __launch_bounds__(256) void qk_prologue_reg_group_kernel(KProblem kp, const __half* q, const __half* k,
                                                                    const float* tab, QKOut o) {
  using S = ProShape<D, 1>;
  constexpr int PARTS = S::PARTS, TASKS = S::TASKS, ROUNDS = S::ROUNDS;
  static_assert(PARTS == 6 && ROUNDS == 2, "six chunks per token, two rounds");
  __shared__ float red[4];
  const int blk = blockIdx.x, h = blockIdx.y;
  const int b = blockIdx.z >> 1, tensor = blockIdx.z & 1;
  const __half* x = tensor ? k : q;

  float v[ROUNDS][32];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r)
#pragma unroll
    for (int e = 0; e < 32; ++e) v[r][e] = 0.f;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int task = threadIdx.x + 256 * r;
    const int tok = task / PARTS, c = task - tok * PARTS;
    const int g = c >> 1, hf = c & 1;
    const int tg = blk * kBlock + tok;
    if (task < TASKS && tg < kp.L) {   // (task < TASKS is wave-uniform)
    // dims [32 hf, 32 hf + nv) of the group are real (nv even; <= 0: none)
    const int nv = kp.split[g] - 32 * hf;
    const long long row = (long long)b * kp.sb + (long long)h * kp.sh + (long long)tg * kp.sl + kp.off[g] + 32 * hf;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(x + row);   // even element offset: 4-byte aligned
    uint32_t raw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) raw[i] = (2 * i < nv) ? src[i] : 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const __half2 hv = *reinterpret_cast<const __half2*>(&raw[i]);
      v[r][2 * i] = __low2float(hv);
      v[r][2 * i + 1] = __high2float(hv);
    }
    if (tg >= kp.prefix) {   // video token: RoPE of the group's pairs 16 hf + i
      const int idx = tg - kp.prefix, hw = kp.Hh * kp.W;
      int t, hq;
      if (kp.L <= (1 << 22)) {   // uniform
        t = quot_small(idx, hw);
        hq = quot_small(idx - t * hw, kp.W);
      } else {
        t = idx / hw;
        hq = (idx - t * hw) / kp.W;
      }
      const int pos = g == 0 ? t : g == 1 ? hq : idx - t * hw - hq * kp.W;
      const int npos = g == 0 ? kp.T : g == 1 ? kp.Hh : kp.W;
      // cos of pair 16 hf + i of axis g at byte oc + 4 i of the table, its sin
      // npos npair[g] floats further
      const uint32_t oc = 4u * (uint32_t)(kp.tab_off[g] + pos * kp.npair[g] + 16 * hf);
      const uint32_t os = oc + 4u * (uint32_t)(npos * kp.npair[g]);
      const char* tb = reinterpret_cast<const char*>(tab);
      float cv[16], sv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        cv[i] = 1.f;
        sv[i] = 0.f;
        if (2 * i < nv) {
          cv[i] = *reinterpret_cast<const float*>(tb + oc + 4u * i);
          sv[i] = *reinterpret_cast<const float*>(tb + os + 4u * i);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float x0 = v[r][2 * i], x1 = v[r][2 * i + 1];
        v[r][2 * i] = fsub_rn(fmul_rn(x0, cv[i]), fmul_rn(x1, sv[i]));
        v[r][2 * i + 1] = fadd_rn(fmul_rn(x0, sv[i]), fmul_rn(x1, cv[i]));
      }
    }
    }
  }
  rotate_quantize<D, 1>(kp, o, b, h, blk, tensor, v, red);
}

// RoPE only, into a dense fp16 copy (the input of the whole-call FP16 path).
template <int D>
__global__ __launch_bounds__(256) void rope_copy_kernel(KProblem kp, const __half* x, const float* tab,
                                                        __half* dst) {
  __shared__ float Y[kBlock][D + 4];
  __shared__ int coord[kBlock][3];
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  load_block_to_lds<D>(kp, x, b, h, blk, Y);
  rope_lds<D>(kp, tab, blk, Y, coord);
  __syncthreads();
  store_rope_copy<D>(kp, b, h, blk, Y, dst);
}


hipError_t launch_rope_tables(const KProblem& kp, float* tab, uint32_t* zero_u32, int n_zero, double phase,
                              hipStream_t s) {
  int entries = 0;
  entries += kp.T * kp.npair[0] + kp.Hh * kp.npair[1] + kp.W * kp.npair[2];
  const int n = entries > n_zero ? entries : n_zero;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, kp, tab, zero_u32, n_zero, phase);
  return hipGetLastError();
}

hipError_t launch_qk_prologue(const KProblem& kp, const __half* q, const __half* k, const float* tab,
                              const QKOut& o, hipStream_t s) {
  dim3 grid(kp.NB, kp.H, 2 * kp.B);
  bool even_pairs = true;
  for (int a = 0; a < 3; ++a) even_pairs = even_pairs && kp.off[a] % 2 == 0 && kp.split[a] % 2 == 0;
  const bool reg_path = even_pairs && kp.rotation != 1;
  if (reg_path) {
    const bool extra = o.q_rope != nullptr || o.k_rope != nullptr || o.q_bsum != nullptr || o.k_bsum != nullptr;
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, kp, q, k, tab, o); };
    const bool r0 = kp.rotation == 0;
    if (kp.D == 128)
      r0 ? (extra ? go(qk_prologue_reg_kernel<128, 0, true>) : go(qk_prologue_reg_kernel<128, 0, false>))
         : (extra ? go(qk_prologue_reg_kernel<128, 2, true>) : go(qk_prologue_reg_kernel<128, 2, false>));
    else
      r0 ? (extra ? go(qk_prologue_reg_kernel<64, 0, true>) : go(qk_prologue_reg_kernel<64, 0, false>))
         : (extra ? go(qk_prologue_reg_kernel<64, 2, true>) : go(qk_prologue_reg_kernel<64, 2, false>));
    return hipGetLastError();
  }
  if (even_pairs && kp.rotation == 1 && o.q_rope == nullptr && o.k_rope == nullptr && o.q_bsum == nullptr &&
      o.k_bsum == nullptr) {
    if (kp.D == 128)
      hipLaunchKernelGGL((qk_prologue_reg_group_kernel<128>), grid, dim3(256), 0, s, kp, q, k, tab, o);
    else
      hipLaunchKernelGGL((qk_prologue_reg_group_kernel<64>), grid, dim3(256), 0, s, kp, q, k, tab, o);
    return hipGetLastError();
  }
  if (kp.D == 128 && kp.rotation == 0)
    hipLaunchKernelGGL((qk_prologue_kernel<128, 0>), grid, dim3(256), 0, s, kp, q, k, tab, o);
  else if (kp.D == 128 && kp.rotation == 1)
    hipLaunchKernelGGL((qk_prologue_kernel<128, 1>), grid, dim3(256), 0, s, kp, q, k, tab, o);
  else if (kp.D == 64 && kp.rotation == 0)
    hipLaunchKernelGGL((qk_prologue_kernel<64, 0>), grid, dim3(256), 0, s, kp, q, k, tab, o);
  else if (kp.D == 64 && kp.rotation == 1)
    hipLaunchKernelGGL((qk_prologue_kernel<64, 1>), grid, dim3(256), 0, s, kp, q, k, tab, o);
  else if (kp.D == 128 && kp.rotation == 2)
    hipLaunchKernelGGL((qk_prologue_kernel<128, 2>), grid, dim3(256), 0, s, kp, q, k, tab, o);
  else if (kp.D == 64 && kp.rotation == 2)
    hipLaunchKernelGGL((qk_prologue_kernel<64, 2>), grid, dim3(256), 0, s, kp, q, k, tab, o);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_rope_copy(const KProblem& kp, const __half* x, const float* tab, __half* dst, hipStream_t s) {
  dim3 grid(kp.NB, kp.H, kp.B);
  if (kp.D == 128)
    hipLaunchKernelGGL((rope_copy_kernel<128>), grid, dim3(256), 0, s, kp, x, tab, dst);
  else if (kp.D == 64)
    hipLaunchKernelGGL((rope_copy_kernel<64>), grid, dim3(256), 0, s, kp, x, tab, dst);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace rotattn
