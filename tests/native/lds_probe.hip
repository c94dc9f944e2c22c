// LDS access-pattern probe for gfx950: one kernel per pattern, each wave
// issuing the same 64-lane LDS instruction over and over at the addresses the
// GEMM kernels use for their fragment reads and slab stores. Run it under
//   rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS ...
// and divide the per-kernel counters by the instruction count to get the LDS
// cycles (and bank-conflict cycles) one such instruction costs.
//
// Patterns (addresses in floats inside one slab, lane l = 32 h + l32):
//  * 128-bit fragment reads of a k-contiguous slab, [lines][BK] with 16-byte
//    chunk c of line r stored at c ^ swz(r): the direct-to-LDS kernels'
//    permutation (swz = (r >> 2) & 3 for BK = 16, (r >> 1) & 7 for BK = 32,
//    r & 15 beyond), the earlier one ((r >> 1) & 3, r & 7), and none;
//  * 128-bit fragment reads of the register-staged kernels' padded slabs
//    [lines][BK + 4];
//  * 32-bit reads in pairs 32 lines apart (ds_read2_b32) of a line-contiguous
//    slab [BK][lines] and of its padded form [BK][lines + 4];
//  * 128-bit slab stores: linear, the register-staged kernels' k-contiguous
//    stores (4 or 8 lanes per line) into padded rows, and the direct kernels'
//    register-path store into swizzled rows.
// Every address stays inside a 64 KiB shared array; the host checks this for
// every pattern and lane before any launch.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

typedef float f4 __attribute__((ext_vector_type(4)));

enum Kind { READ128, READ2_32, WRITE128 };

struct Pattern {
  const char* name;
  Kind kind;
};

constexpr Pattern kPatterns[] = {
    {"read128 linear", READ128},
    {"read128 k-contiguous BK=16, swizzle (r>>2)&3 (direct kernels)", READ128},
    {"read128 k-contiguous BK=16, swizzle (r>>1)&3 (earlier)", READ128},
    {"read128 k-contiguous BK=16, no swizzle", READ128},
    {"read128 k-contiguous BK=32, swizzle (r>>1)&7 (direct kernels)", READ128},
    {"read128 k-contiguous BK=32, swizzle r&7 (earlier)", READ128},
    {"read128 k-contiguous BK=128, swizzle r&15 (direct kernels)", READ128},
    {"read128 k-contiguous BK=128, swizzle r&7 (earlier)", READ128},
    {"read128 padded rows BK=16 (stride 20, register-staged)", READ128},
    {"read128 padded rows BK=32 (stride 36, register-staged)", READ128},
    {"read2_b32 line-contiguous, 256 lines (direct kernels)", READ2_32},
    {"read2_b32 line-contiguous padded, 256+4 lines (register-staged)", READ2_32},
    {"write128 linear", WRITE128},
    {"write128 register-staged k-contiguous BK=16 (4 lanes per line, stride 20)", WRITE128},
    {"write128 register-staged k-contiguous BK=32 (8 lanes per line, stride 36)", WRITE128},
    {"write128 direct kernels' register path BK=16 (swizzle (r>>2)&3)", WRITE128},
};
constexpr int kNumPatterns = sizeof(kPatterns) / sizeof(kPatterns[0]);

__host__ __device__ inline int pattern_address(int p, int lane) {
  const int l32 = lane & 31, h = lane >> 5;
  switch (p) {
    case 0: return 4 * lane;
    case 1: return 16 * l32 + 4 * (h ^ ((l32 >> 2) & 3));
    case 2: return 16 * l32 + 4 * (h ^ ((l32 >> 1) & 3));
    case 3: return 16 * l32 + 4 * h;
    case 4: return 32 * l32 + 4 * (h ^ ((l32 >> 1) & 7));
    case 5: return 32 * l32 + 4 * (h ^ (l32 & 7));
    case 6: return 128 * l32 + 4 * (h ^ (l32 & 15));
    case 7: return 128 * l32 + 4 * (h ^ (l32 & 7));
    case 8: return 20 * l32 + 4 * h;
    case 9: return 36 * l32 + 4 * h;
    case 10: return 4 * h * 256 + l32;
    case 11: return 4 * h * 260 + l32;
    case 12: return 4 * lane;
    case 13: return 20 * (lane / 4) + 4 * (lane % 4);
    case 14: return 36 * (lane / 8) + 4 * (lane % 8);
    case 15: return 16 * (lane / 4) + 4 * ((lane % 4) ^ (((lane / 4) >> 2) & 3));
  }
  return 0;
}

constexpr int kLdsFloats = 16384;  // 64 KiB
constexpr int kShift = 1024;       // floats; eight shifted copies of each pattern
constexpr int kSpan = 40;          // floats beyond an address a pattern may touch (read2 reaches +32, +1)

template <int P>
__global__ void __launch_bounds__(256) probe(float* out, int iters) {
  __shared__ __attribute__((aligned(16))) float lds[kLdsFloats];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int a = pattern_address(P, lane);
  constexpr Kind kind = kPatterns[P].kind;
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (kind == WRITE128) {
    for (int it = 0; it < iters; ++it) {
      const int o = a + ((it + wave) & 7) * kShift;
      *reinterpret_cast<f4*>(lds + o) = acc + (float)it;
    }
    __syncthreads();
    acc = *reinterpret_cast<const f4*>(lds + a);
  } else {
    for (int it = 0; it < iters; ++it) {
      const int o = a + ((it + wave) & 7) * kShift;
      if constexpr (kind == READ2_32) {
        acc.x += lds[o];
        acc.y += lds[o + 32];
      } else {
        acc += *reinterpret_cast<const f4*>(lds + o);
      }
    }
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc.x + acc.y + acc.z + acc.w;
}

template <int P>
bool run_all(float* out, int blocks, int iters) {
  if constexpr (P < kNumPatterns) {
    hipLaunchKernelGGL(probe<P>, dim3(blocks), dim3(256), 0, 0, out, iters);
    if (hipDeviceSynchronize() != hipSuccess) return false;
    printf("pattern %2d: %s\n", P, kPatterns[P].name);
    fflush(stdout);
    return run_all<P + 1>(out, blocks, iters);
  }
  return true;
}

int main() {
  for (int p = 0; p < kNumPatterns; ++p)
    for (int l = 0; l < 64; ++l) {
      const int a = pattern_address(p, l);
      if (a < 0 || a + kSpan + 7 * kShift > kLdsFloats ||
          (kPatterns[p].kind != READ2_32 && a % 4 != 0)) {
        fprintf(stderr, "pattern %d lane %d: address %d out of range or misaligned\n", p, l, a);
        return 1;
      }
    }
  const int blocks = 1024, iters = 256;
  float* out = nullptr;
  if (hipMalloc(&out, sizeof(float) * blocks * 256) != hipSuccess) return 1;
  const bool ok = run_all<0>(out, blocks, iters);
  (void)hipFree(out);
  return ok ? 0 : 1;
}
