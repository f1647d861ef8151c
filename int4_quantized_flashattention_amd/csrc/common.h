// Shared device/host definitions of the rotattn HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace rotattn {

constexpr int kBlock = 64;   // tokens per quantization block and per flash key block

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef short v2s16 __attribute__((ext_vector_type(2)));

// Everything a kernel needs to know about the problem, passed by value.
struct KProblem {
  int B, H, L, D, Dp, Lp, NB;
  int T, Hh, W, prefix;
  int split[3], off[3], npair[3];
  int rotation;
  long long sb, sh, sl;      // element strides of q, k, v, out
  float tau;
  double base;
  int tab_off[3];            // float offset of each axis's cos table; sin follows after n_pos*npair floats
  int tab_floats;            // total floats of all tables
  // the mergeable rotation (rotation 2): a fixed angle added to every RoPE
  // pair's angle, and its float cos/sin for the pairs of text tokens
  double pair_phase;
  float pair_c, pair_s;
};

__device__ __forceinline__ float fmul_rn(float a, float b) { return __fmul_rn(a, b); }
__device__ __forceinline__ float fadd_rn(float a, float b) { return __fadd_rn(a, b); }
__device__ __forceinline__ float fsub_rn(float a, float b) { return __fsub_rn(a, b); }
__device__ __forceinline__ float fdiv_rn(float a, float b) { return __fdiv_rn(a, b); }

// LDS stage of one 64-key block in the INT4 attention kernel, and the byte image
// of it in HBM that the kernel copies with direct-to-LDS loads: 64 K rows of
// DP/32 FP6 E2M3 operand slots and DV V channel rows of two slots, 24 bytes of
// packed values each. Each slot is split into its first 16 bytes, in a plane
// of 16-byte entries, and its last 8, in a plane of 8-byte entries (the
// operand is one 16-byte and one 8-byte LDS read). K slot s of key row r (dims
// [32 s, +32)) and V slot hh of channel row ch (the 32 keys of lane half hh)
// sit at the kvd_* offsets below. The slot permutations put the 16 (32) rows
// that one 16-byte (8-byte) read serves per LDS cycle in distinct banks of the
// 64 (an XOR with a row bit or two for two or four slots per row, a rotation
// by one every 8 or 16 rows for six), and keep rows 32 apart (tiles of 32
// channels) at a constant distance. The image is padded to a multiple of 4096
// bytes, so each thread of a 256-thread workgroup copies the same number of
// 16-byte pieces.
__host__ __device__ constexpr int kv_image_bytes(int DP, int DV) {
  return (kBlock * (DP / 32) * 24 + DV * 48 + 4095) / 4096 * 4096;
}
__host__ __device__ constexpr int kvd_perm(int S, int r, int s, int shift) {
  // shift: 3 for the 16-byte plane, 4 for the 8-byte plane (two or six slots);
  // four slots use the two row bits above shift - 1
  return S == 2 ? (s ^ ((r >> shift) & 1)) : S == 4 ? (s ^ ((r >> (shift - 1)) & 3)) : (s + ((r >> shift) & 1)) % S;
}
__host__ __device__ constexpr int kvd_ka(int DP, int r, int s) { return (r * (DP / 32) + kvd_perm(DP / 32, r, s, 3)) * 16; }
__host__ __device__ constexpr int kvd_kb(int DP, int r, int s) {
  return kBlock * (DP / 32) * 16 + (r * (DP / 32) + kvd_perm(DP / 32, r, s, 4)) * 8;
}
__host__ __device__ constexpr int kvd_va(int DP, int ch, int hh) {
  return kBlock * (DP / 32) * 24 + (ch * 2 + (hh ^ ((ch >> 3) & 1))) * 16;
}
__host__ __device__ constexpr int kvd_vb(int DP, int DV, int ch, int hh) {
  return kBlock * (DP / 32) * 24 + DV * 32 + (ch * 2 + (hh ^ ((ch >> 4) & 1))) * 8;
}
// physical piece of logical 16-byte piece c in row r: c ^ kv_swz(row bytes, r)
__host__ __device__ constexpr int kv_swz(int row_bytes, int r) {
  return row_bytes == 128 ? (((r >> 1) & 7) ^ ((r & 1) << 2)) : (((r >> 1) & 3) ^ ((r >> 3) & 1));
}

// FP16 path: the V^T image of one (b, h, 64-key block) that fp16_vt_kernel
// writes: D rows (channels) of 64 halves (128 bytes), the keys in the order in
// which the P operand of the FP16 P.V product holds them, the 16-byte pieces
// of row ch XOR-permuted by kv_swz(128, ch).
__host__ __device__ constexpr int f16_vt_bytes(int D) { return 128 * D; }

// A row that mixes both paths finishes its FP16 tiles inside the INT4 kernel
// when its head has at most this many flagged K blocks; a head with more has
// its INT4 partial results merged by the FP16 kernel, which stages the K/V
// blocks through LDS.
constexpr unsigned kInlineMaxFlags = 16;

// s_waitcnt that waits until at most N vector-memory operations of this wave
// are outstanding (expcnt and lgkmcnt left alone; gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}
// Direct-to-LDS copies (lds_copy16_s below): lane l's 16 bytes land at LDS
// byte address m0 + 16 l. Written as inline asm
// rather than the builtin so that the compiler does not make LDS reads wait
// for them: once the stage loop wraps around it can no longer tell which stage
// a builtin copy writes and waits for every copy in flight. The callers order
// copies and reads with explicit vmcnt waits and barriers. No register output:
// the copy writes LDS only, and its address registers are read when it issues.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// A wave-uniform pointer in scalar registers: each 32-bit half goes through
// readfirstlane (whose result is a signed int: cast to uint32_t before
// widening, or the low half would be sign-extended into the high one).
__device__ __forceinline__ uint64_t uniform_ptr(const void* p) {
  const uint64_t a = (uint64_t)p;
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
         (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
}
// The copies address a wave-uniform base in scalar registers plus a 32-bit
// per-lane byte offset (no 64-bit vector address per copy); M0 is set without
// saving it (declared clobbered).
__device__ __forceinline__ void lds_copy16_s(uint64_t base, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(m0), "v"(voff), "s"(base)
               : "memory", "m0");
}

// Workgroup barrier without a memory fence: LDS stages are filled by
// direct-to-LDS loads whose completion the caller has already waited for.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Byte i of a byte array that no thread writes during the kernel, for a
// wave-uniform base and i, read through the scalar unit: the dword-aligned
// word holding the byte is loaded (it stays inside the 4-byte granule of a
// valid byte) and the byte shifted out. The address goes through
// readfirstlane so that the load is scalar even where the compiler cannot
// prove it uniform. A vector load here would share the vmcnt counter with the
// direct-to-LDS copies in flight and wait for all of them.
__device__ __forceinline__ uint32_t uniform_byte(const uint8_t* base, int i) {
  const uint64_t addr = reinterpret_cast<uintptr_t>(base) + (uint64_t)(int64_t)i;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
  typedef const __attribute__((address_space(4))) uint32_t* const_u32p;
  const uint32_t w = *reinterpret_cast<const_u32p>(((uint64_t)hi << 32) | (lo & ~3u));
  return (w >> (8 * (lo & 3u))) & 0xFFu;
}

// The same reads from a base already made uniform by uniform_ptr, with a
// wave-uniform index: the address is formed in scalar registers, with no
// readfirstlane per access.
__device__ __forceinline__ uint32_t uniform_byte_u(uint64_t base, int i) {
  const uint64_t addr = base + (uint64_t)(int64_t)i;
  typedef const __attribute__((address_space(4))) uint32_t* const_u32p;
  const uint32_t w = *reinterpret_cast<const_u32p>(addr & ~3ull);
  return (w >> (8 * ((uint32_t)addr & 3u))) & 0xFFu;
}
__device__ __forceinline__ uint32_t uniform_word_u(uint64_t base, int i) {
  typedef const __attribute__((address_space(4))) uint32_t* const_u32p;
  return *reinterpret_cast<const_u32p>(base + 4ull * (uint64_t)(int64_t)i);
}

// Maximum for attention scores and running maxima (finite or -inf): the
// IEEE maximum, which gfx950 computes with v_maximum3_f32 and no extra
// instructions, where fmaxf's NaN rules make the compiler add a
// canonicalizing max before most two-input maxima. (A NaN score, possible
// only from non-finite inputs, propagates.) Nested calls fuse into
// three-input instructions.
__device__ __forceinline__ float smax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float smax3(float a, float b, float c) { return smax(smax(a, b), c); }

__device__ __forceinline__ float wave_max(float v) {
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

}  // namespace rotattn

// Launchers (host side), one per kernel family; defined next to the kernels.
namespace rotattn {
struct QKOut {
  uint8_t* q_codes; uint8_t* k_codes;
  float* q_scale; float* k_scale;
  uint8_t* q_flag; uint8_t* k_flag;
  uint32_t* head_kflag;
  __half* q_rope; __half* k_rope;
  float* q_bsum; float* k_bsum;   // optional 64-token block sums of the RoPE'd rows [B*H][NB][D]
};
struct VOut {
  uint8_t* v_codes; float* v_scale; int32_t* v_colsum;
};
struct AttnArgs {
  const uint8_t* q_codes; const uint8_t* k_codes;
  const float* q_scale; const float* k_scale;
  const uint8_t* q_flag; const uint8_t* k_flag;
  const uint32_t* head_kflag;
  const uint8_t* head_mask;     // [B*H] or null
  const uint8_t* v_codes; const float* v_scale;
  const uint8_t* kv_image;      // [B*H][NB] LDS images of the K/V blocks (kv_image_bytes each)
  const uint8_t* f16_vt;        // [B*H][NB] V^T blocks of the FP16 path (f16_vt_bytes(D) each)
  const uint32_t* block_mask;   // block-sparse: [B*H][ceil(NB/2)][mask_words] key-block bits per 128-row query block
  int mask_words;               // ceil(NB / 32)
  const __half* q_rope; const __half* k_rope; const __half* v;   // FP16 path inputs
  __half* out;
  float* part_o; float* part_m; float* part_l;   // INT4 partials of split rows [B][H][Lp][D], [B][H][Lp]
  bool route;                   // block routing possible (tau finite)
  // dump
  const int32_t* units; int n_units;
  int32_t* d_acc; int8_t* d_pq; int32_t* d_pv; float* d_m;
  float* d_p15;                 // optional: the float32 15 P each P code is rounded from
};

hipError_t launch_rope_tables(const KProblem& kp, float* tab, uint32_t* zero_u32, int n_zero, double phase,
                              hipStream_t s);
hipError_t launch_qk_prologue(const KProblem& kp, const __half* q, const __half* k, const float* tab,
                              const QKOut& o, hipStream_t s);
hipError_t launch_rope_copy(const KProblem& kp, const __half* x, const float* tab, __half* dst, hipStream_t s);
hipError_t launch_vquant(const KProblem& kp, const __half* v, uint32_t* absmax_bits, const VOut& o, hipStream_t s);
hipError_t launch_kv_image(const KProblem& kp, const AttnArgs& a, uint8_t* image, hipStream_t s);
hipError_t launch_int4_attention(const KProblem& kp, const AttnArgs& a, bool dump, hipStream_t s);
hipError_t launch_block_topn(const KProblem& kp, const float* q_bsum, const float* k_bsum, int topn, int sink_rows,
                             int sink_cols, uint32_t* mask, hipStream_t s);
constexpr int kMaxMaskBlocks = 16384;   // largest NB the block-mask builder takes (L <= 1048576)
constexpr int kMaskQBlock = 128;        // query rows per block-sparse mask row (one INT4 workgroup)
hipError_t launch_fp16_vt(const KProblem& kp, const __half* v, uint8_t* image, hipStream_t s);
// which rows the FP16 kernel takes
enum Fp16Rows : int {
  kFp16Routed = 0,     // rows that run whole on FP16 and the merges of INT4 partials
  kFp16WholeCall = 1,  // every row
  kFp16FullOnly = 2,   // rows that run whole on FP16 (masked heads, flagged Q blocks)
  kFp16MergeOnly = 3,  // the merges of INT4 partials (rows that mix both paths in heads with many flagged K blocks)
};
hipError_t launch_fp16_attention(const KProblem& kp, const AttnArgs& a, Fp16Rows rows, hipStream_t s);
}  // namespace rotattn
