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
//  * S^T = K Q^T with v_mfma_f32_32x32x64_f8f6f4 on FP6 E2M3 operands: the
//    Q/K codes in [-7, 7] are exact in E2M3 and the float32 sums of their
//    products are exact integers, so this is the integer Q.K^T, delivered as
//    floats (no int-to-float conversion per score). K codes are the A operand
//    (rows = keys), Q codes the B operand (columns = queries). Each lane then
//    owns one query column and 16 of the 32 keys of a 32 x 32 tile, so the
//    row max and row sum are in-lane plus one exchange with lane ^ 32, and the
//    P codes are already laid out as the B operand of the next product.
//  * O^T = V^T P^T with the same instruction, again on FP6 E2M3 operands: V
//    codes (A, rows = channels; in [-7, 7], exact in E2M3) times the P codes
//    pq + 8 = rne(15 P) in [0, 15] (B), all 32 of a lane from one
//    v_cvt_scalef32_2xpk16_fp6_f32: as E2M3 such a code n is exactly n * 2^-3,
//    so the float32 result is 2^-3 sum (pq + 8) v, exact; the zero-point
//    correction rides inside it, as sum (pq + 8) v = sum pq v + 8 colsum(v)
//    (integer identity). FP6 on both sides takes half the matrix-core cycles
//    of FP8. The float accumulator is rescaled in place when a row max grows.
//  * A pre-pass expands each key block once into the exact LDS image of one
//    pipeline stage: every 24-byte FP6 operand slot (32 K codes of one key,
//    or 32 V codes of one channel) split into a 16-byte and an 8-byte plane,
//    with slots permuted per row so that the operand reads of a wave meet no
//    bank twice on the 64-bank LDS. The loop copies images into LDS with
//    direct-to-LDS loads, three stages deep at D = 128 (four at D = 64).
//  * Block-sparse instances (RainFusion2.0, section 3.1 mask M) visit only the
//    key blocks the workgroup's mask row keeps.
#include "common.h"

#include <climits>
#include <type_traits>

namespace rotattn {

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// FP6 E2M3 bits (sign, 2 exponent bits with bias 1, 3 mantissa bits) of a
// 4-bit two's-complement code in [-7, 7]: every such integer is exact in E2M3
// (7 = 1.75 * 2^2), so the FP6 matrix path also multiplies the codes exactly.
__device__ __forceinline__ uint32_t e2m3_of_code(uint32_t nib) {
  const uint32_t mag = ((nib & 8u) ? 16u - nib : nib) & 7u;   // -8 never occurs for Q/K codes
  return ((uint32_t)(0x1E1C1A1814100800ull >> (8 * mag)) & 0x3Fu) | ((nib & 8u) ? 0x20u : 0u);
}
// 16 packed bytes (32 codes in dim order) -> the 24-byte FP6 operand of those
// 32 values: value i in bits [6 i, 6 i + 6) of six little-endian dwords
__device__ __forceinline__ void e2m3_pack32(uint4 p, uint32_t (&o)[6]) {
  const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
  for (int k = 0; k < 6; ++k) o[k] = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t v = e2m3_of_code((w[i >> 3] >> (4 * (i & 7))) & 15u);
    const int bit = 6 * i, k = bit >> 5, sh = bit & 31;
    o[k] |= v << sh;
    if (sh > 26) o[k + 1] |= v >> (32 - sh);
  }
}

// The 16 V code bytes of one channel and lane half hh (byte 8 s + 4 w + b holds
// key 32 s + 16 w + 4 hh + b in its low nibble, that key + 8 in its high one)
// -> the 24-byte FP6 operand whose element 2 v + s is the key of S^T value v
// of half s (32 s + 8 (v / 4) + 4 hh + v % 4): the element order in which
// v_cvt_scalef32_2xpk16_fp6_f32 interleaves its two 16-float sources.
__device__ __forceinline__ void e2m3_pack32_v(uint4 p, uint32_t (&o)[6]) {
  const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
  for (int k = 0; k < 6; ++k) o[k] = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int s = i & 1, v = i >> 1;
    const uint32_t byte = (w[2 * s + (v >> 3)] >> (8 * (v & 3))) & 0xFFu;
    const uint32_t e = e2m3_of_code(((v >> 2) & 1) ? byte >> 4 : byte & 15u);
    const int bit = 6 * i, k = bit >> 5, sh = bit & 31;
    o[k] |= e << sh;
    if (sh > 26) o[k + 1] |= e >> (32 - sh);
  }
}

// Expands one (b, h, key block) into the LDS image the attention kernel copies:
// the packed K codes of its 64 keys become FP6 E2M3 operand slots (one per run
// of 32 dims) and the V codes of each channel two slots (32 keys each, in the
// element order of the P operand), each slot split over the 16- and 8-byte
// planes at its kvd_* offsets.
template <int DP, int DV>
__global__ __launch_bounds__(256) void kv_image_kernel(KProblem kp, const uint8_t* __restrict__ k_codes,
                                                       const uint8_t* __restrict__ v_codes, uint8_t* image) {
  constexpr int QROW = DP / 2, KPK = kBlock * DP / 2, VPK = DV * 32;
  constexpr int IMG = kv_image_bytes(DP, DV);
  const long long u = blockIdx.x;   // (b * H + h) * NB + block
  const long long bh = u / kp.NB;
  const int j = (int)(u - bh * kp.NB);
  uint8_t* dst = image + u * IMG;
  const uint8_t* kg = k_codes + (bh * kp.Lp + (long long)j * kBlock) * QROW;
  const uint8_t* vg = v_codes + u * VPK;
  for (int o = threadIdx.x * 16; o < KPK; o += 256 * 16) {
    const int r = o / QROW, sl = (o - r * QROW) / 16;   // key row, slot
    uint32_t f6[6];
    e2m3_pack32(*reinterpret_cast<const uint4*>(kg + o), f6);
    *reinterpret_cast<uint4*>(dst + kvd_ka(DP, r, sl)) = make_uint4(f6[0], f6[1], f6[2], f6[3]);
    *reinterpret_cast<uint2*>(dst + kvd_kb(DP, r, sl)) = make_uint2(f6[4], f6[5]);
  }
  for (int o = threadIdx.x * 16; o < VPK; o += 256 * 16) {
    const int ch = o >> 5, hh = (o & 31) / 16;   // channel row, lane half
    uint32_t f6[6];
    e2m3_pack32_v(*reinterpret_cast<const uint4*>(vg + o), f6);
    *reinterpret_cast<uint4*>(dst + kvd_va(DP, ch, hh)) = make_uint4(f6[0], f6[1], f6[2], f6[3]);
    *reinterpret_cast<uint2*>(dst + kvd_vb(DP, DV, ch, hh)) = make_uint2(f6[4], f6[5]);
  }
}

// operand format code of FP6 E2M3 in v_mfma_*_f8f6f4 (cbsz / blgp)
constexpr int kFp6 = 2;

// The FP16 tiles of a row that mixes both paths (RotateAttention abstract,
// selective FP16 fallback; tile routing: head mask, Q flag or K flag), in a
// head with few flagged K blocks, run after the row's INT4 loop has
// finished. The online softmax of RainFusion2.0, section 3.1 continues from
// the INT4 state (m, l, o in V's units) over the head's flagged key blocks in
// ascending order: S^T = K Q^T and O^T = V^T P^T with
// v_mfma_f32_32x32x16_f16 on the RoPE'd, unrotated fp16 Q/K and the V^T block
// images of the FP16 path, P rounded to fp16 for the product and l summed
// from the float32 P. Continuing one recurrence from the other's final state
// is the log-sum-exp merge of the two partial results, and the INT4 codes are
// unaffected: that loop's running max saw its own tiles only. The operands are
// read straight from global memory (L2), which suits a few blocks and keeps
// the INT4 loop's registers and LDS; the lanes of rows past L take part with
// clamped rows and store nothing.
template <int DV>
__device__ __forceinline__ void fp16_tiles_of_mixed_row(const KProblem& kp, const AttnArgs& a, int bh, int row,
                                                        int col, int hh, float c0, float& m, float& l,
                                                        v16f (&o)[DV / 32]) {
  constexpr int NC = DV / 16, NCT = DV / 32, VTB = f16_vt_bytes(DV);
  const int L = kp.L, NB = kp.NB;
  const uint64_t kflag_s = uniform_ptr(a.k_flag + (long long)bh * NB);
  const __half* qrow = a.q_rope + ((long long)bh * L + min(row, L - 1)) * DV + 8 * hh;
  const __half* kbase = a.k_rope + (long long)bh * L * DV + 8 * hh;
  const uint8_t* vbase = a.f16_vt + (long long)bh * NB * VTB;
  for (int j = 0; j < NB; ++j) {
    if (uniform_byte_u(kflag_s, j) == 0) continue;
    v16f sacc[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[s][v] = 0.f;
      const __half* krow = kbase + (long long)min(j * kBlock + 32 * s + col, L - 1) * DV;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const v8h kop = *reinterpret_cast<const v8h*>(krow + 16 * c);
        const v8h qop = *reinterpret_cast<const v8h*>(qrow + 16 * c);
        sacc[s] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kop, qop, sacc[s], 0, 0, 0);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = j * kBlock + 32 * s + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (key >= L) sacc[s][v] = -INFINITY;
        mx = smax(mx, sacc[s][v]);
      }
    {  // the other 32 keys of this query sit in lane ^ 32
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = smax(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // block j holds a key below L, so m_new is finite; alpha = 0 while m = -inf
    const float m_new = smax(m, mx * c0);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[ct][v] *= alpha;
    l *= alpha;
    m = m_new;
    v8h pop[2][2];
    float ps = 0.f;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[s][v], c0, -m));
        ps += p;
        pop[s][v >> 3][v & 7] = (_Float16)p;
      }
    l += ps + __shfl_xor(ps, 32);
    const uint8_t* vblk = vbase + (long long)j * VTB;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int ch = ct * 32 + col;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int pc = 2 * (2 * s + u) + hh;   // logical 16-byte piece: the P operand's keys
          const v8h vop = *reinterpret_cast<const v8h*>(vblk + ch * 128 + 16 * (pc ^ kv_swz(128, ch)));
          o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop, pop[s][u], o[ct], 0, 0, 0);
        }
    }
  }
}

// One workgroup = NW waves = 32*NW query rows of one (b, h). Per key block of
// 64, the block's LDS image (FP6 K rows and FP6 V^T rows, each split into
// 16- and 8-byte planes) arrives in one stage of an NST-stage ring through direct-to-LDS loads issued NST - 1
// blocks ahead; one barrier per block. Every wave computes S^T of its 32
// queries (FP6 products), the online softmax and P codes in registers, and
// O^T on the FP6 matrix path into a float32 accumulator kept at the running
// max, rescaled only when some row max of the wave grows.
// SPARSE: block-sparse attention (RainFusion2.0, section 3.1: Q_i K_j^T and
// P_ij V_j are skipped where M_ij = 0), with one mask row per 128-row query
// block: the loop visits only the key blocks that row keeps.
// ROUTE: the instance for calls with block routing (tau finite), which can
// meet rows that mix both paths: in a head with few flagged K blocks such a
// row finishes its FP16 tiles here after its INT4 loop
// (fp16_tiles_of_mixed_row); in a head with more it writes its INT4 partial
// result for the FP16 kernel to merge. The other instances never meet such
// rows and keep their registers for the loop.
template <int DP, int DV, int NW, int NST, int OCC, bool DUMP, bool SPARSE, bool ROUTE>
__global__ __launch_bounds__(NW * 64, OCC) void int4_attn_kernel(KProblem kp, AttnArgs a, float c0, float log2_15) {
  constexpr int NT = NW * 64;
  constexpr int NC = DP / 64;              // 64-deep slices of the rotated head dim (one FP6 product each)
  constexpr int NCT = DV / 32;             // 32-channel output tiles
  constexpr int QROW = DP / 2;             // packed code bytes per token
  constexpr int IMG = kv_image_bytes(DP, DV);   // one LDS stage = one block's image
  constexpr int NDMA = IMG / (NT * 16);    // 16-byte direct-to-LDS loads per thread per block
  constexpr int NVM = NDMA;                // vector-memory instructions per wave per block
  static_assert(IMG % (NT * 16) == 0, "a stage must split evenly over the workgroup");
  static_assert(NST == 3 || NST == 4, "three or four LDS stages");
  // One LDS array per stage, always indexed by a compile-time stage number:
  // the compiler then knows that reads of one stage cannot alias the
  // direct-to-LDS copies into another and does not wait for those copies.
  __shared__ __attribute__((aligned(16))) uint8_t stg0[IMG];
  __shared__ __attribute__((aligned(16))) uint8_t stg1[IMG];
  __shared__ __attribute__((aligned(16))) uint8_t stg2[IMG];
  __shared__ __attribute__((aligned(16))) uint8_t stg3[NST == 4 ? IMG : 16];
  auto stage = [&](auto s_tag) __attribute__((always_inline)) -> uint8_t* {
    constexpr int S = decltype(s_tag)::value;
    if constexpr (S == 0) return stg0;
    else if constexpr (S == 1) return stg1;
    else if constexpr (S == 2) return stg2;
    else return stg3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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
    // 1D grid over (b, h, 128-row tile); workgroups are dealt round-robin to
    // the 8 XCDs. Without FP16 routing each XCD gets a contiguous run of
    // (b, h, tile), so one head's K/V stream stays in one XCD's L2 (6% faster
    // on block-sparse problems, neutral on dense ones). With routing, whole
    // heads may have no INT4 work: the plain order spreads every head over all
    // XCDs so that none idles (18% faster on the mixed-precision workload).
    const int ntiles = (L + 32 * NW - 1) / (32 * NW);
    const int bid = blockIdx.x;
    int logical = bid;
    if (!(a.route || a.head_mask != nullptr)) {
      const int total = kp.B * kp.H * ntiles;
      const int xcd = bid & 7, slot = bid >> 3;
      const int per = total >> 3, extra = total & 7;   // XCD x gets per + (x < extra) items
      logical = xcd * per + min(xcd, extra) + slot;
    }
    const int bhl = logical / ntiles;
    b = bhl / kp.H;
    h = bhl - b * kp.H;
    row_base = (logical - bhl * ntiles) * (32 * NW);
  }
  // workgroup-uniform: keep them (and every pointer derived from them) in
  // scalar registers
  b = __builtin_amdgcn_readfirstlane(b);
  h = __builtin_amdgcn_readfirstlane(h);
  row_base = __builtin_amdgcn_readfirstlane(row_base);
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

  // Q codes of this lane's query (column) as FP6 E2M3: slice c, lane half hh
  // holds dims [64 c + 32 hh, +32) (the K rows are read with the same split).
  // The FP6 product uses the first six dwords of each operand.
  v8i qop[NC];
  float cq = 0.f;
  if (work) {
    const uint8_t* qrow = a.q_codes + ((long long)bh * Lp + wrow + col) * QROW;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint32_t f6[6];
      e2m3_pack32(*reinterpret_cast<const uint4*>(qrow + 32 * c + 16 * hh), f6);
      qop[c] = v8i{(int)f6[0], (int)f6[1], (int)f6[2], (int)f6[3], (int)f6[4], (int)f6[5], 0, 0};
    }
    cq = fmul_rn(a.q_scale[bh * NB + qblk], c0);
  }

  // wave-uniform bases of the key-block flags and of the mask row (0: none)
  const uint64_t kflag_s = a.route ? uniform_ptr(a.k_flag + (long long)bh * NB) : 0ull;
  // Block-sparse: the bit row (words of 32 key blocks) of the 128-row query
  // block this workgroup covers; every wave processes exactly the key blocks
  // the loop visits.
  const int MW = a.mask_words;
  uint64_t mrow_s = 0;
  if constexpr (SPARSE)
    mrow_s = uniform_ptr(a.block_mask + ((long long)bh * ((NB + 1) / 2) + row_base / kMaskQBlock) * MW);
  // the next key block at or after j that this path takes (NB if none); the
  // result is wave-uniform and formed from scalar loads, which keeps the loop
  // control in scalar registers
  auto next_block = [&](int j) __attribute__((always_inline)) {
    if constexpr (SPARSE) {
      if (j >= NB) return NB;
      int w = j >> 5;
      uint32_t bits = uniform_word_u(mrow_s, w) & (~0u << (j & 31));
      while (bits == 0) {
        if (++w >= MW) return NB;
        bits = uniform_word_u(mrow_s, w);
      }
      j = 32 * w + __builtin_ctz(bits);
      return j < NB ? j : NB;
    } else {
      if (kflag_s != 0ull)
        while (j < NB && uniform_byte_u(kflag_s, j) != 0) ++j;   // FP16 tile: the other path takes it
      return j;
    }
  };
  // Block j's image goes to LDS stage `stage` with NDMA direct-to-LDS loads per
  // thread: thread t copies bytes 16t + 4096i of the image, and the hardware
  // writes lane l's 16 bytes at the wave's LDS base + 16 l.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint8_t* img = a.kv_image + (long long)bh * NB * IMG;   // wave-uniform
  const int toff = tid * 16;                                     // this thread's piece of every round
  // The block's K scale is read through the scalar unit when it is needed.
  const float* kscale = a.k_scale + (long long)bh * NB;
  // Per-thread byte offsets of the pieces stay in registers for the whole
  // loop; the block's image base goes in scalar registers.
  uint32_t voffs[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) voffs[i] = (uint32_t)(toff + i * NT * 16);
  const uint64_t img_s = uniform_ptr(img), ksc_s = uniform_ptr(kscale);
  auto dma_block = [&](int j, auto s_tag) __attribute__((always_inline)) {
    const uint64_t src = img_s + (uint64_t)j * IMG;
    const uint32_t dst = lds_addr(stage(s_tag)) + wave_u * 1024;
#pragma unroll
    for (int i = 0; i < NDMA; ++i) lds_copy16_s(src, voffs[i], dst + i * NT * 16);
  };

  // O^T accumulates on the FP6 matrix path in float32. The V codes are E2M3
  // (exact integers), and the P code n = pq + 8 is the E2M3 value n * 2^-3
  // (a subnormal below 8), so each block adds 2^-3 * sum (pq + 8) v exactly.
  // o is kept at the running max: when a row max of the wave grows it is
  // rescaled in place.
  float m_run = -INFINITY;
  float l15 = 0.f;                 // row sum of 15 P (lane-partial), at m_run
  v16f o[NCT];                     // 2^-3 * sum (pq + 8) v, at m_run
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[ct][v] = 0.f;

  // LDS offsets of this lane's operand pieces: K row `col` (and col + 32, the
  // same permutation) at logical pieces 4c + 2hh and 4c + 2hh + 1 (dims
  // [64 c + 32 hh, +32)); V channel row ct*32 + col (the same permutation for
  // every ct) at logical piece 2*hh + s.
  // kA/kB: the 16- and 8-byte parts of K row col's slot for slice c (row
  // col + 32 lies dKA further, its 8-byte part at kB1); vA/vB: V channel row
  // col's slot, tile ct at vA + ct * 1024 and vB[ct]. All from the stage base.
  constexpr int dKA = 32 * (DP / 32) * 16;
  int kA[NC], kB[NC], kB1[NC], vA, vB[NCT];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    kA[c] = kvd_ka(DP, col, 2 * c + hh);
    kB[c] = kvd_kb(DP, col, 2 * c + hh);
    kB1[c] = kB[c] + 32 * (DP / 32) * 8;
  }
  vA = kvd_va(DP, col, hh);
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) vB[ct] = kvd_vb(DP, DV, col, hh) + ct * 512;
  // Each operand is a 16-byte and an 8-byte LDS read that must land in six
  // consecutive registers. Two 8-byte reads from one base register get paired
  // into a single read2 instruction, which then needs register moves; an
  // opaque base register of its own for every 8-byte read (of K row col + 32
  // and of each V tile) keeps them apart.
#pragma unroll
  for (int c = 0; c < NC; ++c) asm volatile("" : "+v"(kB1[c]));
#pragma unroll
  for (int ct = 1; ct < NCT; ++ct) asm volatile("" : "+v"(vB[ct]));

  // S^T of the block in `stage` (the integer q.k as exact floats), as two
  // 32-key halves, on the FP6 matrix path (E2M3 codes, no block scaling)
  v16f s0, s1;   // S^T of the block in the softmax
  auto qk = [&](const uint8_t* Ks, v16f& d0, v16f& d1) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < 16; ++v) { d0[v] = 0.f; d1[v] = 0.f; }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      // the 24 bytes of the slot: a full first piece and half of the second
      const v4i a0l = *reinterpret_cast<const v4i*>(Ks + kA[c]);
      const v2i a0h = *reinterpret_cast<const v2i*>(Ks + kB[c]);
      const v4i a1l = *reinterpret_cast<const v4i*>(Ks + kA[c] + dKA);
      const v2i a1h = *reinterpret_cast<const v2i*>(Ks + kB1[c]);
      const v8i a0 = v8i{a0l[0], a0l[1], a0l[2], a0l[3], a0h[0], a0h[1], 0, 0};
      const v8i a1 = v8i{a1l[0], a1l[1], a1l[2], a1l[3], a1h[0], a1h[1], 0, 0};
      d0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, qop[c], d0, kFp6, kFp6, 0, 0, 0, 0);
      d1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, qop[c], d1, kFp6, kFp6, 0, 0, 0, 0);
    }
  };

  // Row max, rescale, P codes and P.V of block j (its S^T is in s0/s1, its V in `stage`).
  auto softmax_pv = [&](auto ragged_tag, const uint8_t* Ks, int j) __attribute__((always_inline)) {
    constexpr bool kRagged = decltype(ragged_tag)::value;
    // c = float(float(sq c0) sk)
    // the block's K scale through the scalar unit (uniform address)
    typedef const __attribute__((address_space(4))) float* const_f32p;
    const float sk = *reinterpret_cast<const_f32p>(ksc_s + 4ull * (uint64_t)j);
    const float cs = fmul_rn(cq, sk);
    const int key0 = j * kBlock;
    float mx;
    if (!kRagged) {
      // two interleaved max3 chains over the 32 values of this lane
      float ma = smax3(s0[0], s1[0], s0[2]);
      float mb = smax3(s0[1], s1[1], s0[3]);
#pragma unroll
      for (int v = 2; v < 14; v += 2) {
        ma = smax3(ma, s1[v], s0[v + 2]);
        mb = smax3(mb, s1[v + 1], s0[v + 3]);
      }
      mx = smax(smax3(ma, mb, s1[14]), s1[15]);
    } else {
      mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int k0 = key0 + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (k0 < L) mx = fmaxf(mx, s0[v]);
        if (k0 + 32 < L) mx = fmaxf(mx, s1[v]);
      }
    }
    {  // the other 32 keys of this query sit in lane ^ 32
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = smax(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // max over the block of acc * c = (max acc) * c, as c >= 0 (acc is an exact integer)
    const float m_new = smax(m_run, fmul_rn(mx, cs));
    const bool flush = DUMP || __ballot(m_new > m_run) != 0ull;
    if (flush) {
      // alpha = 2^(m_old - m_new): 0 before the first block, 1 where the row max did not grow
      const float alpha = exp2_hw(fsub_rn(m_run, m_new));
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[ct][v] *= alpha;
      l15 *= alpha;
      m_run = m_new;
    }
    // 15 P = 2^(acc c - (m - log2 15)); its rne is the code pq + 8. All 32
    // codes of the lane come from one v_cvt_scalef32_2xpk16_fp6_f32, which
    // converts 15P / 2^3 to E2M3 with round-to-nearest-even: the E2M3 grid
    // below 2 is exactly the multiples of 2^-3, so each element is
    // rne(15P) * 2^-3, whose six bits read as an integer are rne(15P).
    // Element 2 v + s of the result is value v of half s.
    const float nm15 = -fsub_rn(m_run, log2_15);
    if (DUMP && wrow + col < L) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = key0 + 32 * s + 8 * (v >> 2) + 4 * hh + (v & 3);
          a.d_acc[((long long)unit_idx * kBlock + 32 * wave + col) * Lp + key] = (int)(s == 0 ? s0[v] : s1[v]);
        }
    }
    if constexpr (!kRagged && !DUMP) {
      // full block: every exponent first (in place, S^T is not needed after
      // this), then every exp2, so that the two run as independent streams
#pragma unroll
      for (int v = 0; v < 16; ++v) { s0[v] = fmaf(s0[v], cs, nm15); s1[v] = fmaf(s1[v], cs, nm15); }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int v = 0; v < 16; ++v) { s0[v] = exp2_hw(s0[v]); s1[v] = exp2_hw(s1[v]); }
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float t0 = fmaf(s0[v], cs, nm15), t1 = fmaf(s1[v], cs, nm15);
        if (kRagged) {
          const int key = key0 + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (key >= L) t0 = -INFINITY;
          if (key + 32 >= L) t1 = -INFINITY;
        }
        s0[v] = exp2_hw(t0);
        s1[v] = exp2_hw(t1);
      }
    }
    if (DUMP && a.d_p15 != nullptr && wrow + col < L) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = key0 + 32 * s + 8 * (v >> 2) + 4 * hh + (v & 3);
          a.d_p15[((long long)unit_idx * kBlock + 32 * wave + col) * Lp + key] = s == 0 ? s0[v] : s1[v];
        }
    }
    float ls0 = s0[0], ls1 = s1[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) { ls0 += s0[v]; ls1 += s1[v]; }
    l15 += ls0 + ls1;
    const auto p6 = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(s0, s1, 8.0f);
    if (DUMP && wrow + col < L) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = key0 + 32 * s + 8 * (v >> 2) + 4 * hh + (v & 3);
          const int bit = 6 * (2 * v + s), k = bit >> 5, sh = bit & 31;
          uint32_t e = (uint32_t)p6[k] >> sh;
          if (sh > 26) e |= (uint32_t)p6[k + 1] << (32 - sh);
          a.d_pq[((long long)unit_idx * kBlock + 32 * wave + col) * Lp + key] = (int8_t)((int)(e & 63u) - 8);
        }
    }
    // O^T += V^T (pq + 8)^T: the zero-point correction rides inside the product
    const v8i pb = v8i{(int)p6[0], (int)p6[1], (int)p6[2], (int)p6[3], (int)p6[4], (int)p6[5], 0, 0};
    // raised wave priority while this wave issues its matrix products (P.V
    // here, S^T of the next block after it), so the matrix cores are fed
    // promptly while the other waves of the SIMD run their softmax
    if constexpr (!kRagged) __builtin_amdgcn_s_setprio(1);
    const long long r = (long long)unit_idx * kBlock + 32 * wave + col;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      // the 24 bytes of channel row ct * 32 + col's slot for this lane half
      const v4i vl = *reinterpret_cast<const v4i*>(Ks + vA + ct * 1024);
      const v2i vh = *reinterpret_cast<const v2i*>(Ks + vB[ct]);
      const v8i va = v8i{vl[0], vl[1], vl[2], vl[3], vh[0], vh[1], 0, 0};
      if constexpr (DUMP) {
        // this block's sum alone, to expose the integers sum (pq + 8) v
        v16f z;
#pragma unroll
        for (int v = 0; v < 16; ++v) z[v] = 0.f;
        const v16f blk = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, z, kFp6, kFp6, 0, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          o[ct][v] += blk[v];
          if (wrow + col < L) {
            const int ch = ct * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
            a.d_pv[(r * NB + j) * DV + ch] = (int)(blk[v] * 8.0f);
          }
        }
      } else {
        o[ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, o[ct], kFp6, kFp6, 0, 0, 0, 0);
      }
    }
    if (DUMP && wrow + col < L && hh == 0) a.d_m[r * NB + j] = m_run;
  };

  // Software pipeline over the key blocks this path takes (ascending), with an
  // NST-stage LDS ring filled by direct-to-LDS loads. q[0..NST-1] are the next
  // blocks to process. Entering the iteration for block q[0]: S^T(q[0]) is in
  // s0/s1, q[1] is in LDS, q[2..NST-2] are in flight. The iteration first
  // starts the copy of q[NST-1] into the stage q[0]'s predecessor used, runs
  // the softmax of q[0] (vector ALUs), issues P.V(q[0]) and S^T(q[1]) on the
  // matrix cores, waits for q[2]'s copy and ends with one barrier. Only the
  // last block can be ragged; it is taken after the loop.
  const int nfull = L / kBlock;
  int q[NST];
  q[0] = next_block(0);
#pragma unroll
  for (int i = 1; i < NST; ++i) q[i] = (q[i - 1] < NB) ? next_block(q[i - 1] + 1) : NB;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  if (q[0] < NB) dma_block(q[0], I0());
  if (q[1] < NB) dma_block(q[1], I1());
  if (NST == 4 && q[2] < NB) dma_block(q[2], I2());
  // q[0] and q[1] must have landed; with four stages q[2] may stay in flight
  if (DUMP || NST == 3 || q[2] >= NB) wait_vmcnt<0>();
  else wait_vmcnt<NVM>();
  stage_barrier();
  if (q[0] < NB && work) qk(stage(I0()), s0, s1);
  // one iteration with q[0] in stage S
  auto iter = [&](auto s_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(s_tag)::value;
    using S1 = std::integral_constant<int, (S + 1) % NST>;
    using SL = std::integral_constant<int, (S + NST - 1) % NST>;   // the previous block's stage
    const bool issued = q[NST - 1] < NB;
    if (issued) dma_block(q[NST - 1], SL());
    if (work) {
      // S^T of the next block after this block's P.V (stale data when there
      // is no next block: computed, never used)
      softmax_pv(std::integral_constant<bool, false>(), stage(s_tag), q[0]);
      qk(stage(S1()), s0, s1);
      __builtin_amdgcn_s_setprio(0);
    }
    // q[2] must have landed before the next iteration reads it
    if (DUMP || NST == 3 || !issued) wait_vmcnt<0>();
    else wait_vmcnt<NVM>();
    stage_barrier();
#pragma unroll
    for (int i = 0; i < NST - 1; ++i) q[i] = q[i + 1];
    q[NST - 1] = (q[NST - 2] < NB) ? next_block(q[NST - 2] + 1) : NB;
  };
  int st = 0;   // stage of q[0] when the loop ends
  for (;;) {
    if (q[0] >= nfull) { st = 0; break; }
    iter(I0());
    if (q[0] >= nfull) { st = 1; break; }
    iter(I1());
    if (q[0] >= nfull) { st = 2; break; }
    iter(I2());
    if constexpr (NST == 4) {
      if (q[0] >= nfull) { st = 3; break; }
      iter(I3());
    }
  }
  const int j = q[0];
  if (j < NB && work) {
    wait_vmcnt<0>();
    const uint8_t* Ks = st == 0 ? stage(I0()) : st == 1 ? stage(I1()) : st == 2 ? stage(I2()) : stage(I3());
    softmax_pv(std::integral_constant<bool, true>(), Ks, j);
  }

  if (DUMP || !work) return;
  const float l15t = l15 + __shfl_xor(l15, 32);
  const int row = wrow + col;
  const float* svp = a.v_scale + (long long)bh * DV;
  __half* orow = a.out + (long long)b * kp.sb + (long long)h * kp.sh + (long long)row * kp.sl;
  if constexpr (ROUTE && !DUMP && !SPARSE) {
    if (mixed) {
      if (a.head_kflag[bh] <= kInlineMaxFlags) {
        // the INT4 partial in V's units: O = 2^3 o s_v / 15 and l = l15 / 15,
        // at m_run; then the FP16 tiles
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[ct][v] *= svp[ct * 32 + 8 * (v >> 2) + 4 * hh + (v & 3)] * (8.0f / 15.0f);
        float l = l15t * (1.0f / 15.0f);
        fp16_tiles_of_mixed_row<DV>(kp, a, bh, row, col, hh, c0, m_run, l, o);
        if (row >= L) return;
        const float inv = 1.0f / l;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int ch = ct * 32 + 8 * g + 4 * hh;
            __half hv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) hv[e] = __float2half_rn(o[ct][4 * g + e] * inv);
            *reinterpret_cast<uint2*>(orow + ch) = *reinterpret_cast<const uint2*>(hv);
          }
        return;
      }
      // many flagged K blocks: the INT4 partial (O s_v / 15 with O = 2^3 o;
      // m; l = l15 / 15) for the FP16 kernel to merge
      if (row >= L) return;
      float* po = a.part_o + ((long long)bh * Lp + row) * DV;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ch = ct * 32 + 8 * g + 4 * hh;
          float4 f;
          f.x = o[ct][4 * g + 0] * (svp[ch + 0] * (8.0f / 15.0f));
          f.y = o[ct][4 * g + 1] * (svp[ch + 1] * (8.0f / 15.0f));
          f.z = o[ct][4 * g + 2] * (svp[ch + 2] * (8.0f / 15.0f));
          f.w = o[ct][4 * g + 3] * (svp[ch + 3] * (8.0f / 15.0f));
          *reinterpret_cast<float4*>(po + ch) = f;
        }
      if (hh == 0) {
        a.part_m[(long long)bh * Lp + row] = m_run;
        a.part_l[(long long)bh * Lp + row] = l15t * (1.0f / 15.0f);
      }
      return;
    }
  }
  if (row >= L) return;
  // out = O (s_v / 15) / l with O = 2^3 o and l = l15 / 15 (a sparse row
  // that keeps no key block gets zeros)
  const float inv = (SPARSE && l15t == 0.f) ? 0.f : 8.0f / l15t;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int ch = ct * 32 + 8 * g + 4 * hh;
      __half hv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[e] = __float2half_rn(o[ct][4 * g + e] * svp[ch + e] * inv);
      *reinterpret_cast<uint2*>(orow + ch) = *reinterpret_cast<const uint2*>(hv);
    }
}

// Launch shape per rotated head dim. Four waves per workgroup (32 query rows
// each), so that independent workgroups share a CU and one's softmax overlaps
// another's matrix work. Workgroups per CU (kOcc): three at D' = 128, where the
// registers (at most 168 per lane) and three LDS rings fit, which measured 10%
// faster than two workgroups with four stages and the next block's S^T issued
// early; two elsewhere (the D' = 192 rings do not fit three times; D = 64
// reaches four workgroups per CU through its register count anyway). Stages:
// three at D = 128 (with the 12 KB image of D' = 128 four fit, but measured
// 0.6% slower), else as many as kOcc rings fit in the 160 KB of LDS.
template <int DP, int DV>
struct Shape {
  static constexpr int kWaves = 4;
  static constexpr int kOcc = (DP == 128) ? 3 : 2;
  static constexpr int kStages =
      (DV == 128) ? 3 : ((kOcc * 4 * (kv_image_bytes(DP, DV) + 256) + 1024 <= 160 * 1024) ? 4 : 3);
};

template <int DP, int DV, bool SPARSE>
static void launch_int4_s(const KProblem& kp, const AttnArgs& a, bool dump, float c0, float l15, hipStream_t s) {
  using S = Shape<DP, DV>;
  constexpr int W = S::kWaves, NS = S::kStages, OC = S::kOcc;
  if (dump) {
    hipLaunchKernelGGL((int4_attn_kernel<DP, DV, W, NS, OC, true, SPARSE, false>), dim3(a.n_units), dim3(W * 64),
                       0, s, kp, a, c0, l15);
  } else {
    const int ntiles = (kp.L + 32 * W - 1) / (32 * W);
    dim3 grid(ntiles * kp.H * kp.B);
    // the routed instance: two workgroups per CU at D' = 128, where three
    // would make it spill; at D' = 192 held to the registers of three
    constexpr int OCR = (DP == 128) ? 2 : (DP == 192 && DV == 128) ? 3 : OC;
    if (!SPARSE && a.route)
      hipLaunchKernelGGL((int4_attn_kernel<DP, DV, W, NS, OCR, false, SPARSE, !SPARSE>), grid, dim3(W * 64), 0, s,
                         kp, a, c0, l15);
    else
      hipLaunchKernelGGL((int4_attn_kernel<DP, DV, W, NS, OC, false, SPARSE, false>), grid, dim3(W * 64), 0, s, kp,
                         a, c0, l15);
  }
}

template <int DP, int DV>
static hipError_t launch_int4_t(const KProblem& kp, const AttnArgs& a, bool dump, float c0, float l15,
                                hipStream_t s) {
  if (a.block_mask != nullptr)
    launch_int4_s<DP, DV, true>(kp, a, dump, c0, l15, s);
  else
    launch_int4_s<DP, DV, false>(kp, a, dump, c0, l15, s);
  return hipGetLastError();
}

template <int DP, int DV>
static hipError_t launch_kv_image_t(const KProblem& kp, const AttnArgs& a, uint8_t* image, hipStream_t s) {
  const long long units = (long long)kp.B * kp.H * kp.NB;
  hipLaunchKernelGGL((kv_image_kernel<DP, DV>), dim3((unsigned)units), dim3(256), 0, s, kp, a.k_codes, a.v_codes,
                     image);
  return hipGetLastError();
}

hipError_t launch_kv_image(const KProblem& kp, const AttnArgs& a, uint8_t* image, hipStream_t s) {
  if (kp.Dp == 128 && kp.D == 128) return launch_kv_image_t<128, 128>(kp, a, image, s);
  if (kp.Dp == 192 && kp.D == 128) return launch_kv_image_t<192, 128>(kp, a, image, s);
  if (kp.Dp == 64 && kp.D == 64) return launch_kv_image_t<64, 64>(kp, a, image, s);
  if (kp.Dp == 192 && kp.D == 64) return launch_kv_image_t<192, 64>(kp, a, image, s);
  return hipErrorInvalidValue;
}

hipError_t launch_int4_attention(const KProblem& kp, const AttnArgs& a, bool dump, hipStream_t s) {
  const float c0 = (float)(std::log2(2.718281828459045) / std::sqrt((double)kp.D));
  const float l15 = (float)std::log2(15.0);
  if (kp.Dp == 128 && kp.D == 128) return launch_int4_t<128, 128>(kp, a, dump, c0, l15, s);
  if (kp.Dp == 192 && kp.D == 128) return launch_int4_t<192, 128>(kp, a, dump, c0, l15, s);
  if (kp.Dp == 64 && kp.D == 64) return launch_int4_t<64, 64>(kp, a, dump, c0, l15, s);
  if (kp.Dp == 192 && kp.D == 64) return launch_int4_t<192, 64>(kp, a, dump, c0, l15, s);
  return hipErrorInvalidValue;
}

}  // namespace rotattn
