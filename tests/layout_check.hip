// Host-side checks of the LDS layouts the attention kernels index (common.h),
// built with hipcc --offload-host-only and run on the CPU by test_layout.py:
//  1. the K/V block image: every byte of every FP6 slot plane lands inside
//     kv_image_bytes, and no two slots overlap;
//  2. LDS banks: for each operand read of the INT4 kernel (K rows col and
//     col + 32, slot 2c + lane half; V channel rows, slot = lane half) and of
//     the FP16 kernel's V^T rows, the lanes one LDS cycle serves (16 for a
//     16-byte read, 32 for an 8-byte read; 64 banks of 4 bytes) touch
//     distinct banks;
//  3. a control: the same reads of an unpermuted layout do conflict, so the
//     bank model is not vacuous.
// Prints one line per check and "ok" at the end; the exit status counts the failures.
#include "common.h"

#include <cstdio>
#include <set>
#include <vector>

using namespace rotattn;

static int conflicts(const int* addr, int bytes) {
  const int group = 256 / bytes;
  int bad = 0;
  for (int g0 = 0; g0 < 64; g0 += group) {
    std::set<int> banks;
    int want = 0;
    for (int l = g0; l < g0 + group; ++l)
      for (int b = 0; b < bytes / 4; ++b) {
        banks.insert((addr[l] / 4 + b) % 64);
        ++want;
      }
    bad += want - (int)banks.size();
  }
  return bad;
}

int main() {
  int fail = 0;
  const int shapes[4][2] = {{128, 128}, {192, 128}, {64, 64}, {192, 64}};
  for (const auto& sh : shapes) {
    const int DP = sh[0], DV = sh[1];
    const int IMG = kv_image_bytes(DP, DV);
    std::vector<int> cover(IMG, 0);
    int outside = 0;
    auto mark = [&](int off, int n) {
      for (int b = 0; b < n; ++b) {
        if (off + b < 0 || off + b >= IMG) ++outside;
        else ++cover[off + b];
      }
    };
    for (int r = 0; r < kBlock; ++r)
      for (int s = 0; s < DP / 32; ++s) {
        mark(kvd_ka(DP, r, s), 16);
        mark(kvd_kb(DP, r, s), 8);
      }
    for (int ch = 0; ch < DV; ++ch)
      for (int hh = 0; hh < 2; ++hh) {
        mark(kvd_va(DP, ch, hh), 16);
        mark(kvd_vb(DP, DV, ch, hh), 8);
      }
    int overlap = 0, used = 0;
    for (int x : cover) {
      overlap += x > 1;
      used += x > 0;
    }
    const int want = kBlock * (DP / 32) * 24 + DV * 48;
    const bool ok = outside == 0 && overlap == 0 && used == want;
    printf("image DP=%d DV=%d bytes=%d used=%d outside=%d overlap=%d %s\n", DP, DV, IMG, used, outside, overlap,
           ok ? "ok" : "FAIL");
    fail += !ok;

    int a[64], bank = 0;
    for (int c = 0; c < DP / 64; ++c)
      for (int half = 0; half < 2; ++half) {
        for (int l = 0; l < 64; ++l) a[l] = kvd_ka(DP, (l & 31) + 32 * half, 2 * c + (l >> 5));
        bank += conflicts(a, 16);
        for (int l = 0; l < 64; ++l) a[l] = kvd_kb(DP, (l & 31) + 32 * half, 2 * c + (l >> 5));
        bank += conflicts(a, 8);
      }
    for (int ct = 0; ct < DV / 32; ++ct) {
      for (int l = 0; l < 64; ++l) a[l] = kvd_va(DP, ct * 32 + (l & 31), l >> 5);
      bank += conflicts(a, 16);
      for (int l = 0; l < 64; ++l) a[l] = kvd_vb(DP, DV, ct * 32 + (l & 31), l >> 5);
      bank += conflicts(a, 8);
    }
    printf("int4 banks DP=%d DV=%d extra_bank_cycles=%d %s\n", DP, DV, bank, bank == 0 ? "ok" : "FAIL");
    fail += bank != 0;

    // control: slots in plain row order
    int ctl = 0;
    for (int l = 0; l < 64; ++l) a[l] = ((l & 31) * (DP / 32) + (l >> 5)) * 16;
    ctl += conflicts(a, 16);
    printf("control DP=%d conflicts=%d %s\n", DP, ctl, ctl > 0 ? "ok" : "FAIL");
    fail += ctl == 0;
  }
  // FP16 kernel: V^T rows of 128 bytes, 16-byte pieces XOR-permuted by kv_swz(128, row)
  for (int D = 64; D <= 128; D += 64) {
    int a[64], bank = 0;
    for (int ct = 0; ct < D / 32; ++ct)
      for (int su = 0; su < 4; ++su) {
        for (int l = 0; l < 64; ++l) {
          const int col = l & 31, hh = l >> 5, row = ct * 32 + col;
          a[l] = row * 128 + 16 * ((2 * su + hh) ^ kv_swz(128, row));
        }
        bank += conflicts(a, 16);
      }
    printf("fp16 vt banks D=%d extra_bank_cycles=%d %s\n", D, bank, bank == 0 ? "ok" : "FAIL");
    fail += bank != 0;
  }
  if (fail == 0) printf("ok\n");
  return fail;
}
