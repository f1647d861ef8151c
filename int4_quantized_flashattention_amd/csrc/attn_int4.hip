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
#include <type_traits>

namespace rotattn {

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Unpacks 16 packed bytes (32 INT4 codes) into 32 int8 bytes (each code times
// 16) in the order the matrix-core operands read them, and stores them to LDS.
__device__ __forceinline__ void store_unpacked(uint8_t* dst, uint4 p) {
  uint4 a, b;
  a.x = nib_lo16(p.x); a.y = nib_hi16(p.x); a.z = nib_lo16(p.y); a.w = nib_hi16(p.y);
  b.x = nib_lo16(p.z); b.y = nib_hi16(p.z); b.z = nib_lo16(p.w); b.w = nib_hi16(p.w);
  reinterpret_cast<uint4*>(dst)[0] = a;
  reinterpret_cast<uint4*>(dst)[1] = b;
}

// One workgroup = NW waves = 32*NW query rows of one (b, h). Per key block of
// 64: the packed K and V codes (prefetched into registers during the previous
// block) are unpacked once into one of two LDS stages, one barrier, then every
// wave runs two S^T tiles, the online softmax and four O^T tiles on the
// matrix cores. O is accumulated in int32 by the matrix cores and folded into
// the float32 accumulator only when some row max of the wave grows (the
// rescale factor is exactly 1 otherwise).
template <int DP, int DV, int NW, bool DUMP>
__global__ __launch_bounds__(NW * 64, 2) void int4_attn_kernel(KProblem kp, AttnArgs a, float c0, float log2_15) {
  constexpr int NT = NW * 64;
  constexpr int NC = DP / 32;              // 32-deep slices of the rotated head dim
  constexpr int NCT = DV / 32;             // 32-channel output tiles
  constexpr int QROW = DP / 2;             // packed code bytes per token
  constexpr int HALF = DP / 4;             // packed code bytes of one lane half
  constexpr int KPK = kBlock * DP / 2;     // packed K bytes per key block
  constexpr int VPK = DV * 32;             // packed V bytes per key block
  constexpr int PK = KPK + VPK;
  constexpr int KROW = DP + 16;            // unpacked K row in LDS (padded)
  constexpr int VROW = 64 + 16;            // unpacked V channel row in LDS (padded)
  constexpr int KST = kBlock * KROW;
  constexpr int STAGE = KST + DV * VROW + 16;   // + the K block scale
  constexpr int NLOAD = (PK + NT * 16 - 1) / (NT * 16);
  __shared__ __attribute__((aligned(16))) uint8_t smem[3 * STAGE];

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
    // 1D grid. Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
    // contiguous run of (b, h, row tile) so that one head's K/V stream stays in
    // one XCD's L2 instead of being fetched by all eight.
    const int ntiles = (L + 32 * NW - 1) / (32 * NW);
    const int total = kp.B * kp.H * ntiles;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    const int per = total >> 3, extra = total & 7;   // XCD x gets per + (x < extra) items
    const int logical = xcd * per + min(xcd, extra) + slot;
    const int bhl = logical / ntiles;
    b = bhl / kp.H;
    h = bhl - b * kp.H;
    row_base = (logical - bhl * ntiles) * (32 * NW);
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

  const uint8_t* kg = a.k_codes + (long long)bh * Lp * QROW;
  const uint8_t* vg = a.v_codes + (long long)bh * NB * VPK;
  const uint8_t* kflag = a.route ? a.k_flag + (long long)bh * NB : nullptr;
  auto next_block = [&](int j) {
    if (kflag != nullptr)
      while (j < NB && kflag[j] != 0) ++j;   // FP16 tile: the other path takes it
    return j;
  };
  // Packed codes of a future block wait in registers; store_stage unpacks
  // them into one of the three LDS stages.
  uint4 pre[NLOAD];
  float sk_pre = 0.f;   // K block scale, carried through LDS with the tile
  auto load_block = [&](int j) {
    if (tid == 0) sk_pre = a.k_scale[bh * NB + j];
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      const int o = (tid + i * NT) * 16;
      // passes that lie wholly inside the K part or the V part need no per-thread test
      const bool allK = (i + 1) * NT * 16 <= KPK;
      const bool allV = i * NT * 16 >= KPK && (i + 1) * NT * 16 <= PK;
      if (allK || (!allV && o < KPK)) pre[i] = *reinterpret_cast<const uint4*>(kg + (long long)j * KPK + o);
      else if (allV || o < PK) pre[i] = *reinterpret_cast<const uint4*>(vg + (long long)j * VPK + (o - KPK));
    }
  };
  auto store_stage = [&](int stage) {
    uint8_t* base = smem + stage * STAGE;
    if (tid == 0) *reinterpret_cast<float*>(base + STAGE - 16) = sk_pre;
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      const int o = (tid + i * NT) * 16;
      const bool allK = (i + 1) * NT * 16 <= KPK;
      const bool allV = i * NT * 16 >= KPK && (i + 1) * NT * 16 <= PK;
      if (allK || (!allV && o < KPK)) {
        const int r = o / QROW, bo = o - (o / QROW) * QROW;
        store_unpacked(base + r * KROW + 2 * bo, pre[i]);
      } else if (allV || o < PK) {
        const int ov = o - KPK, c = ov >> 5, bo = ov & 31;
        store_unpacked(base + KST + c * VROW + 2 * bo, pre[i]);
      }
    }
  };

  // O = o_acc * 2^(m_ref - m_run) + pacc: o_acc holds everything folded so far
  // at a fixed reference max m_ref (per row), pacc the int32 sum since the
  // last fold at the current running max m_run. A fold is one multiply-add
  // per value and leaves o_acc unscaled; the reference moves only when
  // m_run - m_ref exceeds 64 (to keep o_acc far from overflow).
  float m_run = -INFINITY;
  float m_ref = -INFINITY;
  float l15 = 0.f;                 // row sum of 15 P (lane-partial), at m_run
  v16f o_acc[NCT];                 // float32 O (times 16) at m_ref
  v16i pacc[NCT];                  // int32 O (times 16) at m_run since the last fold
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int v = 0; v < 16; ++v) { o_acc[ct][v] = 0.f; pacc[ct][v] = 0; }

  // S^T (times 256) of the block in `stage`, as two 32-key halves
  v16i s0, s1;
  auto qk = [&](int stage) {
    const uint8_t* Ks = smem + stage * STAGE;
#pragma unroll
    for (int v = 0; v < 16; ++v) { s0[v] = 0; s1[v] = 0; }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const v4i a0 = *reinterpret_cast<const v4i*>(Ks + col * KROW + hh * (DP / 2) + 16 * c);
      const v4i a1 = *reinterpret_cast<const v4i*>(Ks + (32 + col) * KROW + hh * (DP / 2) + 16 * c);
      s0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, qop[c], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, qop[c], s1, 0, 0, 0);
    }
  };

  // Row max, rescale, P codes and P.V of block j (its S^T is in s0/s1, its V in `stage`).
  auto softmax_pv = [&](auto ragged_tag, int stage, int j) {
    constexpr bool kRagged = decltype(ragged_tag)::value;
    const uint8_t* Ks = smem + stage * STAGE;
    const uint8_t* Vs = Ks + KST;
    // c = float(float(sq c0) sk); the operands carry a factor 256, folded in exactly
    const float sk = *reinterpret_cast<const float*>(Ks + STAGE - 16);
    const float cs = fmul_rn(fmul_rn(cq, sk), 1.0f / 256.0f);
    const int key0 = j * kBlock;
    int mx;
    if (!kRagged) {
      // two interleaved max3 chains over the 32 values of this lane
      int ma = max(s0[0], s1[0]), mb = max(s0[1], s1[1]);
#pragma unroll
      for (int v = 2; v < 16; v += 2) {
        ma = max(max(ma, s0[v]), s1[v]);
        mb = max(max(mb, s0[v + 1]), s1[v + 1]);
      }
      mx = max(ma, mb);
    } else {
      mx = INT_MIN;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int k0 = key0 + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (k0 < L) mx = max(mx, s0[v]);
        if (k0 + 32 < L) mx = max(mx, s1[v]);
      }
    }
    {  // the other 32 keys of this query sit in lane ^ 32
      const auto sw = __builtin_amdgcn_permlane32_swap(mx, mx, false, false);
      mx = max((int)sw[0], (int)sw[1]);   // the builtin yields unsigned lanes: compare as signed
    }
    // max over the block of float(acc) * c = float(max acc) * c, as c >= 0
    const float m_new = fmaxf(m_run, fmul_rn((float)mx, cs));
    const bool flush = DUMP || __ballot(m_new > m_run) != 0ull;
    if (flush) {
      // fold pacc (at m_run) into o_acc (at m_ref); nothing folded yet before the first block
      const bool first = m_run == -INFINITY;
      const float g = first ? 0.f : exp2_hw(fsub_rn(m_run, m_ref));
      m_ref = first ? m_new : m_ref;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int v = 0; v < 16; ++v) o_acc[ct][v] = fmaf((float)pacc[ct][v], g, o_acc[ct][v]);
      {  // zero the int32 accumulators on the matrix cores (0 x 0 + 0)
        v4i z4;
        v16i z16;
#pragma unroll
        for (int v = 0; v < 4; ++v) z4[v] = 0;
#pragma unroll
        for (int v = 0; v < 16; ++v) z16[v] = 0;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) pacc[ct] = __builtin_amdgcn_mfma_i32_32x32x32_i8(z4, z4, z16, 0, 0, 0);
      }
      l15 *= exp2_hw(fsub_rn(m_run, m_new));
      m_run = m_new;
      if (__ballot(fsub_rn(m_run, m_ref) > 64.f) != 0ull) {
        const float f = exp2_hw(fsub_rn(m_ref, m_run));
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int v = 0; v < 16; ++v) o_acc[ct][v] *= f;
        m_ref = m_run;
      }
    }
    // 15 P = 2^(acc c - (m - log2 15)); its rne is pq + 8, packed by v_cvt_pk_u8_f32
    const float nm15 = -fsub_rn(m_run, log2_15);
    v4i pop[2];
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        uint32_t word = 0;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int v = 4 * kq + bb;
          float t = fmaf((float)(s == 0 ? s0[v] : s1[v]), cs, nm15);
          if (kRagged) {
            const int key = key0 + 32 * s + 8 * kq + 4 * hh + bb;
            if (key >= L) t = -INFINITY;
          }
          const float p15 = exp2_hw(t);
          if (bb & 1) ls1 += p15; else ls0 += p15;
          word = __builtin_amdgcn_cvt_pk_u8_f32(p15, bb, word);
          if (DUMP && wrow + col < L) {
            const int key = key0 + 32 * s + 8 * kq + 4 * hh + bb;
            const long long di = ((long long)unit_idx * kBlock + 32 * wave + col) * Lp + key;
            a.d_acc[di] = (s == 0 ? s0[v] : s1[v]) >> 8;
            a.d_pq[di] = (int8_t)((int)((word >> (8 * bb)) & 0xFFu) - 8);
          }
        }
        pop[s][kq] = (int)word;
      }
    l15 += ls0 + ls1;
    // O^T += V^T (pq + 8)^T: the zero-point correction rides inside the product
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const v4i vop = *reinterpret_cast<const v4i*>(Vs + (ct * 32 + col) * VROW + 32 * hh + 16 * s);
        pacc[ct] = __builtin_amdgcn_mfma_i32_32x32x32_i8(vop, pop[s], pacc[ct], 0, 0, 0);
      }
    }
    if (DUMP && wrow + col < L) {
      const long long r = (long long)unit_idx * kBlock + 32 * wave + col;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int ch = ct * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
          a.d_pv[(r * NB + j) * DV + ch] = pacc[ct][v] >> 4;
        }
      if (hh == 0) a.d_m[r * NB + j] = m_run;
    }
  };

  // Software pipeline over the key blocks this path takes (ascending), with a
  // three-stage LDS ring. Entering the iteration for block j: S^T(j) is in
  // s0/s1, block j+1 is in LDS, the packed codes of block j+2 are in flight.
  // The iteration runs the softmax of block j (vector ALUs), then issues
  // P.V(j) and S^T(j+1) on the matrix cores while it unpacks block j+2 into
  // the stage block j-1 used. One barrier per block. Only the last block can
  // be ragged; it is taken after the loop.
  const int nfull = L / kBlock;
  int j = next_block(0);
  int jn = NB, jnn = NB;
  if (j < NB) {
    load_block(j);
    store_stage(0);
    jn = next_block(j + 1);
    if (jn < NB) {
      load_block(jn);
      store_stage(1);
      jnn = next_block(jn + 1);
      if (jnn < NB) load_block(jnn);
    }
    __syncthreads();
    if (work) qk(0);
  }
  int st = 0;
  while (j < nfull) {
    const int st1 = (st == 2) ? 0 : st + 1;
    const int st2 = (st1 == 2) ? 0 : st1 + 1;
    if (work) {
      softmax_pv(std::integral_constant<bool, false>(), st, j);
      qk(st1);   // stale data when there is no next block: computed, never used
    }
    const int j3 = (jnn < NB) ? next_block(jnn + 1) : NB;
    if (jnn < NB) {
      store_stage(st2);
      if (j3 < NB) load_block(j3);
    }
    __syncthreads();
    st = st1;
    j = jn;
    jn = jnn;
    jnn = j3;
  }
  if (j < NB && work) softmax_pv(std::integral_constant<bool, true>(), st, j);

  if (DUMP || !work) return;
  {  // O = o_acc 2^(m_ref - m_run) + pacc
    const float f = (m_run == -INFINITY) ? 0.f : exp2_hw(fsub_rn(m_ref, m_run));
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) o_acc[ct][v] = fmaf(o_acc[ct][v], f, (float)pacc[ct][v]);
  }
  const float l15t = l15 + __shfl_xor(l15, 32);
  const int row = wrow + col;
  if (row >= L) return;
  const float* svp = a.v_scale + (long long)bh * DV;
  if (!mixed) {
    // out = O (s_v / 15) / l with O = o/16 and l = l15/15
    const float inv = 1.0f / (16.0f * l15t);
    __half* orow = a.out + (long long)b * kp.sb + (long long)h * kp.sh + (long long)row * kp.sl;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = ct * 32 + 8 * g + 4 * hh;
        __half hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = __float2half_rn(o_acc[ct][4 * g + e] * svp[ch + e] * inv);
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
      a.part_l[(long long)bh * Lp + row] = l15t * (1.0f / 15.0f);
    }
  }
}

// waves per workgroup (32 query rows each): four, so that two independent
// workgroups share a CU and one's softmax overlaps the other's matrix work
template <int DP>
constexpr int waves_for() { return 4; }

template <int DP, int DV>
static hipError_t launch_int4_t(const KProblem& kp, const AttnArgs& a, bool dump, float c0, float l15,
                                hipStream_t s) {
  constexpr int kWaves = waves_for<DP>();
  if (dump) {
    hipLaunchKernelGGL((int4_attn_kernel<DP, DV, kWaves, true>), dim3(a.n_units), dim3(kWaves * 64), 0, s, kp, a,
                       c0, l15);
  } else {
    const int ntiles = (kp.L + 32 * kWaves - 1) / (32 * kWaves);
    dim3 grid(ntiles * kp.H * kp.B);
    hipLaunchKernelGGL((int4_attn_kernel<DP, DV, kWaves, false>), grid, dim3(kWaves * 64), 0, s, kp, a, c0, l15);
  }
  return hipGetLastError();
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
