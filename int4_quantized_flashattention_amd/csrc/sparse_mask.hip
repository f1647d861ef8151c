// Block mask of block-sparse attention (RainFusion2.0, sections 3.2
// "Representative Token for Blocks" and 3.4 "First Frame Sink").
//
// Query blocks of 128 rows (one workgroup of the INT4 kernel), key blocks of
// 64 keys (section 3.1 lets b_q and b_k differ). For query block i of head
// (b, h): S_hat[i][j] = q_hat_i . k_hat_j over the block means of the RoPE'd
// Q and K (float32, from the block sums the Q/K prologue writes); the topn key blocks with the largest S_hat (equal scores
// in ascending j) are kept, then every key block holding a first-frame or
// text token is kept, and a query block holding such a token keeps every key
// block. Output: bit j % 32 of word j / 32 of row (bh, i) is 1 when key block
// j is kept; bits at or beyond NB are 0.
#include "common.h"

#include <type_traits>

namespace rotattn {

constexpr int kMaskRows = 8;   // most query blocks per workgroup

// float -> uint32 whose unsigned order is the float order
__device__ __forceinline__ uint32_t sortable(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// One workgroup per (QB consecutive 128-row query blocks, b*H + h), four
// waves. Representative tokens from the 64-token block sums of the Q/K
// prologue: q_hat_i = (sum_{2i} + sum_{2i+1}) / rows, k_hat_j = sum_j / keys
// (IEEE division; a multiply by 2^-6 for full key blocks, which is the same
// value). Scores: lane l of a wave owns key block j = 64 t + l of tile t and
// computes S_hat for every query block of the workgroup as one float32 fma
// chain over the head dim in ascending order. Selection: one wave per query
// block (a radix select of the topn-th largest score, then the ties in
// ascending j). Dynamic LDS: QB * NB scores (as sortable u32 keys), then
// 4 * NB flags.
template <int D>
__global__ __launch_bounds__(256) void block_topn_kernel(KProblem kp, const float* __restrict__ q_bsum,
                                                         const float* __restrict__ k_bsum, int topn, int sink_rows,
                                                         int sink_cols, int QB, uint32_t* mask) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int NB = kp.NB, NQ = (NB + 1) / 2, MW = (NB + 31) / 32;
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem);
  __shared__ uint32_t hist[4][256];
  __shared__ __attribute__((aligned(16))) float qh[kMaskRows][D];

  const long long bh = blockIdx.y;
  const int i0 = blockIdx.x * QB;
  const int nrows = min(QB, NQ - i0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint8_t* sel = smem + (size_t)4 * QB * NB + (size_t)wave * NB;
  const float* qs = q_bsum + bh * NB * D;
  const float* ks = k_bsum + bh * NB * D;

  for (int e = tid; e < kMaskRows * D; e += 256) {   // rows past the workgroup's: zeros (scored, not stored)
    const int r = e / D, d = e - r * D;
    const int i = i0 + r;
    float v = 0.f;
    if (r < nrows) {
      v = qs[(long long)(2 * i) * D + d];
      if (2 * i + 1 < NB) v = fadd_rn(v, qs[(long long)(2 * i + 1) * D + d]);
      v = fdiv_rn(v, (float)min(kMaskQBlock, kp.L - kMaskQBlock * i));
    }
    qh[r][d] = v;
  }
  __syncthreads();
  for (int j = tid; j < NB; j += 256) {
    const float* kj = ks + (long long)j * D;
    const int cnt = min(kBlock, kp.L - kBlock * j);
    float acc[kMaskRows];
#pragma unroll
    for (int r = 0; r < kMaskRows; ++r) acc[r] = 0.f;
    auto chain = [&](auto full_tag) __attribute__((always_inline)) {
      constexpr bool kFull = decltype(full_tag)::value;
#pragma unroll 8
      for (int d = 0; d < D; d += 4) {
        const float4 s4 = *reinterpret_cast<const float4*>(kj + d);
        const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float kv = kFull ? sv[e] * 0.015625f : fdiv_rn(sv[e], (float)cnt);
#pragma unroll
          for (int r = 0; r < kMaskRows; ++r) acc[r] = __builtin_fmaf(qh[r][d + e], kv, acc[r]);
        }
      }
    };
    if (cnt == kBlock) chain(std::true_type());   // every key block but a ragged last one
    else chain(std::false_type());
#pragma unroll
    for (int r = 0; r < kMaskRows; ++r)
      if (r < nrows) keys[(size_t)r * NB + j] = sortable(acc[r]);
  }
  __syncthreads();

  const int n = topn < NB ? topn : NB;
  const int chunk = (NB + 63) / 64;
  const int j0 = lane * chunk, j1 = min(NB, j0 + chunk);
  uint32_t* hw = hist[wave];
  for (int r = wave; r < nrows; r += 4) {   // wave-uniform
    const int i = i0 + r;
    uint32_t* row = mask + (bh * NQ + i) * MW;
    if (i < sink_rows) {   // a sink query block keeps every key block
      for (int w = lane; w < MW; w += 64) {
        const int nb = NB - 32 * w;
        row[w] = nb >= 32 ? 0xFFFFFFFFu : ((1u << nb) - 1u);
      }
      continue;
    }
    const uint32_t* key = keys + (size_t)r * NB;
    // radix select (most significant byte first) of the n-th largest key
    uint32_t prefix = 0, pmask = 0;
    uint32_t need = (uint32_t)n;   // rank of the wanted key among those matching the prefix (1 = largest)
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
      for (int c = 0; c < 4; ++c) hw[4 * lane + c] = 0;
      __builtin_amdgcn_wave_barrier();
      for (int j = lane; j < NB; j += 64)
        if ((key[j] & pmask) == prefix) atomicAdd(&hw[(key[j] >> shift) & 255u], 1u);
      __builtin_amdgcn_wave_barrier();
      // lane l owns bins 252 - 4l .. 255 - 4l (lane 0 the largest digits);
      // count the keys in the bins above each bin, from the top
      uint32_t c[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] = hw[255 - 4 * lane - e];
      const uint32_t mine = c[0] + c[1] + c[2] + c[3];
      uint32_t above = wave_incl_scan(mine) - mine;
      int found = -1;
      uint32_t rest = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (found < 0 && above < need && above + c[e] >= need) { found = 255 - 4 * lane - e; rest = need - above; }
        above += c[e];
      }
      const uint64_t hit = __ballot(found >= 0);
      const int src = __builtin_ctzll(hit);
      const uint32_t digit = (uint32_t)__shfl(found, src);
      need = (uint32_t)__shfl((int)rest, src);
      prefix |= digit << shift;
      pmask |= 255u << shift;
      __builtin_amdgcn_wave_barrier();
    }
    const uint32_t T = prefix;   // the n-th largest key; `need` keys equal to T are kept, lowest j first
    // ties: lane l owns the contiguous range [j0, j1) of j
    uint32_t eq = 0;
    for (int j = j0; j < j1; ++j) eq += (key[j] == T) ? 1u : 0u;
    uint32_t before = wave_incl_scan(eq) - eq;
    for (int j = j0; j < j1; ++j) {
      uint8_t f = 0;
      if (key[j] > T) f = 1;
      else if (key[j] == T) { f = (before < need) ? 1 : 0; ++before; }
      sel[j] = f;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int w = lane; w < MW; w += 64) {
      uint32_t bits = 0;
      for (int e = 0; e < 32; ++e) {
        const int j = 32 * w + e;
        if (j < NB && (sel[j] != 0 || j < sink_cols)) bits |= 1u << e;
      }
      row[w] = bits;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// 128-row query blocks per workgroup: at most kMaskRows, and the scores of a
// workgroup within 48 KB of LDS (three workgroups per CU)
static int mask_rows(int NB) {
  int qb = (49152 - 4 * NB) / (4 * NB);
  return qb < 1 ? 1 : (qb > kMaskRows ? kMaskRows : qb);
}

template <int D>
static hipError_t launch_topn_t(const KProblem& kp, const float* q_bsum, const float* k_bsum, int topn, int sink_rows,
                                int sink_cols, uint32_t* mask, hipStream_t s) {
  const int QB = mask_rows(kp.NB);
  const int NQ = (kp.NB + 1) / 2;
  const size_t lds = (size_t)4 * QB * kp.NB + (size_t)4 * kp.NB;   // scores, then four waves' flags
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&block_topn_kernel<D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((NQ + QB - 1) / QB, kp.B * kp.H);
  hipLaunchKernelGGL((block_topn_kernel<D>), grid, dim3(256), lds, s, kp, q_bsum, k_bsum, topn, sink_rows, sink_cols,
                     QB, mask);
  return hipGetLastError();
}

hipError_t launch_block_topn(const KProblem& kp, const float* q_bsum, const float* k_bsum, int topn, int sink_rows,
                             int sink_cols, uint32_t* mask, hipStream_t s) {
  if (kp.D == 128) return launch_topn_t<128>(kp, q_bsum, k_bsum, topn, sink_rows, sink_cols, mask, s);
  if (kp.D == 64) return launch_topn_t<64>(kp, q_bsum, k_bsum, topn, sink_rows, sink_cols, mask, s);
  return hipErrorInvalidValue;
}

}  // namespace rotattn
