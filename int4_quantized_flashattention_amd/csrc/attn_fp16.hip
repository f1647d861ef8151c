// FP16 flash-attention path: the selective FP16 fallback of RotateAttention
// (arXiv 2607.02584, abstract) for masked heads, flagged Q blocks and whole
// denoising steps, and for the flagged K blocks of rows that mix both paths
// in heads with many flagged K blocks (more than kInlineMaxFlags), whose INT4
// partials it merges by log-sum-exp in its epilogue. (In heads with few, the
// INT4 kernel finishes such rows itself.)
//
// Recurrences: RainFusion2.0, section 3.1 "Blockwise Sparse", in the log2
// domain over key blocks of 64; a tile that belongs to the INT4 path is
// skipped (the block mask M of the same section).
//
// Same work layout as the INT4 kernel: S^T = K Q^T and O^T = V^T P^T with
// v_mfma_f32_32x32x16_f16, one query column per lane, P rounded to fp16 in
// registers as the B operand of the second product, O accumulated in fp32 by
// the matrix cores and rescaled only when a row max of the wave grows. Inputs
// are RoPE'd, unrotated Q/K (fp16, dense) and the caller's fp16 V. K rows go
// straight from HBM into a two-stage LDS ring with direct-to-LDS loads (the
// XOR permutation of their 16-byte pieces is applied to the source
// addresses); V is staged the same way from a pre-pass that writes V^T per
// (b, h, 64-key block) with its keys in the order of the P operand.
#include "common.h"

#include <cmath>

namespace rotattn {

__device__ __forceinline__ float exp2_hw16(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS stage of one key block: 64 K rows of D halves (16-byte pieces
// XOR-permuted per row), then D rows of V^T, 64 halves each (permuted the same
// way as 128-byte rows). 256 * D bytes; the pre-pass writes the V^T half.
template <int D>
__device__ __forceinline__ int f16_kswz(int r) { return D == 128 ? (r & 15) : kv_swz(128, r); }
// key (within the block) whose value sits at position pos of a V^T row: the
// order in which the P operand of the second product holds its keys
__device__ __forceinline__ int f16_key_of_pos(int pos) {
  return (pos & 32) + (pos & 16) + 8 * ((pos >> 2) & 1) + 4 * ((pos >> 3) & 1) + (pos & 3);
}

template <int D>
__global__ __launch_bounds__(256) void fp16_vt_kernel(KProblem kp, const __half* __restrict__ v, uint8_t* image) {
  __shared__ __attribute__((aligned(16))) __half vt[kBlock][D + 8];
  const long long u = blockIdx.x;
  const long long bh = u / kp.NB;
  const int j = (int)(u - bh * kp.NB);
  const int b = (int)(bh / kp.H), h = (int)(bh - (long long)b * kp.H);
  uint8_t* dst = image + u * f16_vt_bytes(D);
  for (int idx = threadIdx.x; idx < kBlock * D / 8; idx += 256) {
    const int r = idx / (D / 8), pc = idx - r * (D / 8);
    const int key = j * kBlock + r;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (key < kp.L)
      val = *reinterpret_cast<const uint4*>(v + (long long)b * kp.sb + (long long)h * kp.sh +
                                            (long long)key * kp.sl + pc * 8);
    *reinterpret_cast<uint4*>(&vt[r][pc * 8]) = val;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < D * 8; idx += 256) {   // (channel, 8-position piece)
    const int ch = idx >> 3, pc = idx & 7;
    __half hv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) hv[e] = vt[f16_key_of_pos(8 * pc + e)][ch];
    *reinterpret_cast<uint4*>(dst + ch * 128 + 16 * (pc ^ kv_swz(128, ch))) = *reinterpret_cast<const uint4*>(hv);
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void fp16_attn_kernel(KProblem kp, AttnArgs a, int rows_sel, float c0) {
  constexpr int NC = D / 16;       // 16-deep slices of the head dim
  constexpr int NCT = D / 32;      // 32-channel output tiles
  constexpr int KROWB = 2 * D, VT0 = 64 * KROWB, VTB = f16_vt_bytes(D);
  constexpr int IMG = VT0 + VTB;
  constexpr int NDK = VT0 / 4096, NDV = VTB / 4096;   // 16-byte copies per thread per stage
  static_assert(VT0 % 4096 == 0 && VTB % 4096 == 0, "a stage must split evenly over the workgroup");
  // one LDS array per stage, indexed by compile-time stage numbers
  __shared__ __attribute__((aligned(16))) uint8_t stg0[IMG];
  __shared__ __attribute__((aligned(16))) uint8_t stg1[IMG];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int L = kp.L, Lp = kp.Lp, NB = kp.NB;
  const int b = blockIdx.z, h = blockIdx.y, bh = b * kp.H + h;
  const int wrow = blockIdx.x * 128 + 32 * wave;
  const bool active = wrow < L;
  const int qblk = wrow / kBlock;
  // per wave: `full` rows take every key block on this path, `mixed` rows the
  // flagged key blocks only (their other blocks ran on the INT4 path)
  bool full = false, mixed = false;
  if (active) {
    full = rows_sel == kFp16WholeCall || (a.head_mask != nullptr && uniform_byte(a.head_mask, bh) != 0) ||
           (a.route && uniform_byte(a.q_flag, bh * NB + qblk) != 0);
    mixed = !full && a.route && a.head_kflag[bh] > kInlineMaxFlags;
    if (rows_sel == kFp16FullOnly) mixed = false;
    if (rows_sel == kFp16MergeOnly) full = false;
  }
  const bool any_full = __builtin_amdgcn_readfirstlane(__syncthreads_or(full)) != 0;
  const bool any_mixed = __builtin_amdgcn_readfirstlane(__syncthreads_or(mixed)) != 0;
  if (!any_full && !any_mixed) return;

  const int row = wrow + col;
  v8h qop[NC];
  if (full || mixed) {
    const __half* qrow = a.q_rope + ((long long)bh * L + (row < L ? row : L - 1)) * D + 8 * hh;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint4 u = *reinterpret_cast<const uint4*>(qrow + 16 * c);
      qop[c] = *reinterpret_cast<const v8h*>(&u);
    }
  }
  // LDS offsets: K row col (and col + 32) at piece 2c + hh (dims [16c + 8hh, +8));
  // V^T row ct*32 + col at piece 4s + 2u + hh
  int koff[NC], voff[4];
#pragma unroll
  for (int c = 0; c < NC; ++c) koff[c] = col * KROWB + 16 * ((2 * c + hh) ^ f16_kswz<D>(col));
#pragma unroll
  for (int su = 0; su < 4; ++su) voff[su] = VT0 + col * 128 + 16 * ((2 * su + hh) ^ kv_swz(128, col));

  // wave-uniform base of the key-block flags (0: no routing)
  const uint64_t kflag_s = a.route ? uniform_ptr(a.k_flag + (long long)bh * NB) : 0ull;
  // key blocks this workgroup visits: all when some row runs whole on this
  // path, else the flagged ones only (wave-uniform, from scalar loads)
  auto next_block = [&](int j) __attribute__((always_inline)) {
    if (!any_full && kflag_s != 0ull)
      while (j < NB && uniform_byte_u(kflag_s, j) == 0) ++j;
    return j;
  };
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // thread tid fills LDS bytes [i * 4096 + 16 * tid, +16) of each stage; for the
  // K half that is row kr[i], physical piece kp_[i], holding logical piece
  // kp_[i] ^ swz(row) of key j * 64 + kr[i] (the last key row stands in past L:
  // those keys are masked out of S)
  // Copies address a wave-uniform base in scalar registers (the key block's
  // first K row, the block's V^T image) plus a 32-bit lane offset within it.
  const uint64_t kbase_s = uniform_ptr(a.k_rope + (long long)bh * L * D);
  const uint64_t vimg_s = uniform_ptr(a.f16_vt + (long long)bh * NB * VTB);
  int krow[NDK];
  uint32_t kcol[NDK], voffs[NDV];
#pragma unroll
  for (int i = 0; i < NDK; ++i) {
    const int o = i * 4096 + tid * 16;
    krow[i] = o / KROWB;
    kcol[i] = (uint32_t)(16 * (((o % KROWB) >> 4) ^ f16_kswz<D>(krow[i])));   // byte offset in the row
  }
#pragma unroll
  for (int i = 0; i < NDV; ++i) voffs[i] = (uint32_t)(tid * 16 + i * 4096);
  auto dma_block = [&](int j, uint8_t* stage_base) __attribute__((always_inline)) {
    const uint32_t dst = lds_addr(stage_base) + wave_u * 1024;
    const uint64_t ksrc = kbase_s + (uint64_t)j * (kBlock * 2 * D);
    const int last = L - 1 - j * kBlock;   // rows past L repeat the last key (masked out of S)
#pragma unroll
    for (int i = 0; i < NDK; ++i) {
      const int r = min(krow[i], last);
      lds_copy16_s(ksrc, (uint32_t)r * (uint32_t)(2 * D) + kcol[i], dst + i * 4096);
    }
    const uint64_t vsrc = vimg_s + (uint64_t)j * VTB;
#pragma unroll
    for (int i = 0; i < NDV; ++i) lds_copy16_s(vsrc, voffs[i], dst + VT0 + i * 4096);
  };

  float m_run = -INFINITY, l_part = 0.f;
  v16f o_acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int v = 0; v < 16; ++v) o_acc[ct][v] = 0.f;

  auto compute = [&](const uint8_t* Ks, int j) __attribute__((always_inline)) {
    v16f sacc[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[s][v] = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const v8h kop = *reinterpret_cast<const v8h*>(Ks + koff[c] + s * 32 * KROWB);
        sacc[s] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kop, qop[c], sacc[s], 0, 0, 0);
      }
    }
    // row max of the raw scores (c0 > 0, so max(S c0) = max(S) c0); keys
    // past L only in the last block
    float mx;
    if (j * kBlock + kBlock > L) {
      const int key0 = j * kBlock;
      mx = -INFINITY;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = key0 + 32 * s + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (key >= L) sacc[s][v] = -INFINITY;
          mx = fmaxf(mx, sacc[s][v]);
        }
    } else {
      // two interleaved max3 chains over the 32 values of this lane
      float ma = smax3(sacc[0][0], sacc[1][0], sacc[0][2]);
      float mb = smax3(sacc[0][1], sacc[1][1], sacc[0][3]);
#pragma unroll
      for (int v = 2; v < 14; v += 2) {
        ma = smax3(ma, sacc[1][v], sacc[0][v + 2]);
        mb = smax3(mb, sacc[1][v + 1], sacc[0][v + 3]);
      }
      mx = smax(smax3(ma, mb, sacc[1][14]), sacc[1][15]);
    }
    {  // the other 32 keys of this query sit in lane ^ 32
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = smax(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float m_new = smax(m_run, mx * c0);
    if (__ballot(m_new > m_run) != 0ull) {   // rescale only when some row max grew
      const float alpha = exp2_hw16(m_run - m_new);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int v = 0; v < 16; ++v) o_acc[ct][v] *= alpha;
      l_part *= alpha;
      m_run = m_new;
    }
    // P = 2^(S c0 - m): exponents first, then the exp2s, as independent streams
    const float nm = -m_run;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[s][v] = fmaf(sacc[s][v], c0, nm);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[s][v] = exp2_hw16(sacc[s][v]);
    __builtin_amdgcn_sched_barrier(0);
    v8h pop[2][2];
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        ps[v & 3] += sacc[s][v];
        pop[s][v >> 3][v & 7] = (_Float16)sacc[s][v];
      }
    l_part += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const v8h vop = *reinterpret_cast<const v8h*>(Ks + voff[2 * s + u] + ct * 32 * 128);
          o_acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop, pop[s][u], o_acc[ct], 0, 0, 0);
        }
  };

  // two-stage ring: entering the iteration for block j, j is in LDS; the
  // iteration starts the copy of the next block into the other stage, computes
  // j, waits for the copy and ends with one barrier
  int j = next_block(0);
  if (j < NB) dma_block(j, stg0);
  wait_vmcnt<0>();
  stage_barrier();
  auto iter = [&](auto s_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(s_tag)::value;
    uint8_t* cur = S == 0 ? stg0 : stg1;
    uint8_t* oth = S == 0 ? stg1 : stg0;
    const int jn = (j + 1 < NB) ? next_block(j + 1) : NB;
    if (jn < NB) dma_block(jn, oth);
    if (full || (mixed && uniform_byte_u(kflag_s, j) != 0)) {
      compute(cur, j);
      __builtin_amdgcn_s_setprio(0);
    }
    wait_vmcnt<0>();
    stage_barrier();
    j = jn;
  };
  while (j < NB) {
    iter(std::integral_constant<int, 0>());
    if (j >= NB) break;
    iter(std::integral_constant<int, 1>());
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
    float4 p1[NCT][4];   // all loads first: the stores below may alias them for the compiler
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) p1[ct][g] = *reinterpret_cast<const float4*>(po + ct * 32 + 8 * g + 4 * hh);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float o1[4] = {p1[ct][g].x, p1[ct][g].y, p1[ct][g].z, p1[ct][g].w};
        __half hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = __float2half_rn((a1 * o1[e] + a2 * o_acc[ct][4 * g + e]) * inv);
        *reinterpret_cast<uint2*>(orow + ct * 32 + 8 * g + 4 * hh) = *reinterpret_cast<const uint2*>(hv);
      }
  }
}

hipError_t launch_fp16_vt(const KProblem& kp, const __half* v, uint8_t* image, hipStream_t s) {
  const unsigned units = (unsigned)((long long)kp.B * kp.H * kp.NB);
  if (kp.D == 128)
    hipLaunchKernelGGL((fp16_vt_kernel<128>), dim3(units), dim3(256), 0, s, kp, v, image);
  else if (kp.D == 64)
    hipLaunchKernelGGL((fp16_vt_kernel<64>), dim3(units), dim3(256), 0, s, kp, v, image);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_fp16_attention(const KProblem& kp, const AttnArgs& a, Fp16Rows rows, hipStream_t s) {
  const float c0 = (float)(std::log2(2.718281828459045) / std::sqrt((double)kp.D));
  dim3 grid((kp.L + 127) / 128, kp.H, kp.B);
  if (kp.D == 128)
    hipLaunchKernelGGL((fp16_attn_kernel<128>), grid, dim3(256), 0, s, kp, a, (int)rows, c0);
  else if (kp.D == 64)
    hipLaunchKernelGGL((fp16_attn_kernel<64>), grid, dim3(256), 0, s, kp, a, (int)rows, c0);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace rotattn
