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
typedef int v16i __attribute__((ext_vector_type(16)));
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
};

__device__ __forceinline__ float fmul_rn(float a, float b) { return __fmul_rn(a, b); }
__device__ __forceinline__ float fadd_rn(float a, float b) { return __fadd_rn(a, b); }
__device__ __forceinline__ float fsub_rn(float a, float b) { return __fsub_rn(a, b); }
__device__ __forceinline__ float fdiv_rn(float a, float b) { return __fdiv_rn(a, b); }

// INT4 nibbles -> int8 lanes scaled by 16: low nibbles of w, then high nibbles of w.
// (w << 4) & 0xF0F0F0F0 moves each low nibble to the top of its byte, keeping its
// sign bit as the byte's sign; w & 0xF0F0F0F0 keeps the high nibbles in place.
__device__ __forceinline__ int nib_lo16(uint32_t w) { return (int)((w << 4) & 0xF0F0F0F0u); }
__device__ __forceinline__ int nib_hi16(uint32_t w) { return (int)(w & 0xF0F0F0F0u); }

// 8 packed bytes (16 codes) -> a 16 x int8 matrix-core operand (each value times 16).
__device__ __forceinline__ v4i unpack16(uint2 p) {
  v4i r;
  r[0] = nib_lo16(p.x);
  r[1] = nib_hi16(p.x);
  r[2] = nib_lo16(p.y);
  r[3] = nib_hi16(p.y);
  return r;
}

// LDS stage of one 64-key block in the INT4 attention kernel, and the byte image
// of it in HBM that the kernel copies with direct-to-LDS loads: 64 K rows of DP
// int8 operand bytes, then DV V channel rows of 64 int8 operand bytes. Within a
// row the 16-byte pieces are permuted by kv_swz so that 8 or 16 consecutive
// rows read at the same logical piece fall in distinct LDS banks. Every size is
// a multiple of 4096 bytes, so each thread of a 256-thread workgroup copies the
// same number of 16-byte pieces.
__host__ __device__ constexpr int kv_kst(int DP) { return kBlock * DP; }
__host__ __device__ constexpr int kv_image_bytes(int DP, int DV) { return kBlock * DP + DV * 64; }
// physical piece of logical 16-byte piece c in row r: c ^ kv_swz(row bytes, r)
__host__ __device__ constexpr int kv_swz(int row_bytes, int r) {
  return row_bytes == 128 ? (((r >> 1) & 7) ^ ((r & 1) << 2)) : (((r >> 1) & 3) ^ ((r >> 3) & 1));
}

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
  const __half* q_rope; const __half* k_rope; const __half* v;   // FP16 path inputs
  __half* out;
  float* part_o; float* part_m; float* part_l;   // INT4 partials of mixed rows [B][H][Lp][D], [B][H][Lp]
  bool route;                   // block routing possible (tau finite)
  // dump
  const int32_t* units; int n_units;
  int32_t* d_acc; int8_t* d_pq; int32_t* d_pv; float* d_m;
};

hipError_t launch_rope_tables(const KProblem& kp, float* tab, uint32_t* zero_u32, int n_zero, hipStream_t s);
hipError_t launch_qk_prologue(const KProblem& kp, const __half* q, const __half* k, const float* tab,
                              const QKOut& o, hipStream_t s);
hipError_t launch_rope_copy(const KProblem& kp, const __half* x, const float* tab, __half* dst, hipStream_t s);
hipError_t launch_vquant(const KProblem& kp, const __half* v, uint32_t* absmax_bits, const VOut& o, hipStream_t s);
hipError_t launch_kv_image(const KProblem& kp, const AttnArgs& a, uint8_t* image, hipStream_t s);
hipError_t launch_int4_attention(const KProblem& kp, const AttnArgs& a, bool dump, hipStream_t s);
hipError_t launch_fp16_attention(const KProblem& kp, const AttnArgs& a, bool whole_call, hipStream_t s);
}  // namespace rotattn
