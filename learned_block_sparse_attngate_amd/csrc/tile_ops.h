// LDS tile machinery shared by the attention kernels (prefill and decode):
// 64-key K / V tiles copied HBM -> LDS with buffer_load ... lds under an XOR
// chunk swizzle, and the operand reads that feed v_mfma_f32_32x32x16_bf16
// (K rows as the A operand of S^T = K Q^T, V^T through transposing reads as
// the A operand of O^T = V^T P^T). Internal to the kernel translation units.
#pragma once

#include <stdint.h>

#include <type_traits>
#include <utility>

#include "seer_device.h"

namespace seer {

constexpr int kBufferWord3 = 0x00020000; // gfx9-family raw buffer resource, dword 3

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>)
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// 16-byte-chunk XOR swizzles (chunk index within a row of the LDS tile).
//  K: the 32x32x16 A-operand read has 16 consecutive keys at one logical chunk.
//  V: a ds_read_b64_tr_b16 reads 8 consecutive keys x 4 consecutive chunks.
template <int D> __device__ __forceinline__ int swz_k(int row) { return row & (D / 8 - 1); }
template <int D> __device__ __forceinline__ int swz_v(int row) { return D == 128 ? 4 * (row & 3) : 4 * (row & 1); }

// Workgroup barrier without a memory fence. Inside the tile pipeline the
// copies into LDS are ordered with explicit vmcnt waits and the LDS reads
// with lgkmcnt waits; a fence would also wait for every copy in flight.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }


// LDS reads outside the compiler's view of the copies in flight; each waits
// for its own result before returning.
__device__ __forceinline__ uint32_t lds_read_u16(uint32_t addr) {
  uint32_t v;
  asm volatile("ds_read_u16 %0, %1\n s_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ uint32_t lds_read_u32(uint32_t addr) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n s_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)p));
}

// K operands of one tile for S^T = K Q^T: kr[2 ks + mt] holds keys 32 mt + l32,
// dims 16 ks + 8 hl .. +7. Waits for its own LDS reads before returning.
template <int D>
__device__ __forceinline__ void read_k_tile(const uint32_t (&kaddr)[D / 16], u32x4_t (&kr)[D / 8]) {
  if constexpr (D == 128) {
    asm volatile(
        "ds_read_b128 %0, %16\n ds_read_b128 %1, %16 offset:8192\n"
        "ds_read_b128 %2, %17\n ds_read_b128 %3, %17 offset:8192\n"
        "ds_read_b128 %4, %18\n ds_read_b128 %5, %18 offset:8192\n"
        "ds_read_b128 %6, %19\n ds_read_b128 %7, %19 offset:8192\n"
        "ds_read_b128 %8, %20\n ds_read_b128 %9, %20 offset:8192\n"
        "ds_read_b128 %10, %21\n ds_read_b128 %11, %21 offset:8192\n"
        "ds_read_b128 %12, %22\n ds_read_b128 %13, %22 offset:8192\n"
        "ds_read_b128 %14, %23\n ds_read_b128 %15, %23 offset:8192\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kr[0]), "=&v"(kr[1]), "=&v"(kr[2]), "=&v"(kr[3]), "=&v"(kr[4]), "=&v"(kr[5]), "=&v"(kr[6]),
          "=&v"(kr[7]), "=&v"(kr[8]), "=&v"(kr[9]), "=&v"(kr[10]), "=&v"(kr[11]), "=&v"(kr[12]), "=&v"(kr[13]),
          "=&v"(kr[14]), "=&v"(kr[15])
        : "v"(kaddr[0]), "v"(kaddr[1]), "v"(kaddr[2]), "v"(kaddr[3]), "v"(kaddr[4]), "v"(kaddr[5]),
          "v"(kaddr[6]), "v"(kaddr[7])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %8\n ds_read_b128 %1, %8 offset:4096\n"
        "ds_read_b128 %2, %9\n ds_read_b128 %3, %9 offset:4096\n"
        "ds_read_b128 %4, %10\n ds_read_b128 %5, %10 offset:4096\n"
        "ds_read_b128 %6, %11\n ds_read_b128 %7, %11 offset:4096\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kr[0]), "=&v"(kr[1]), "=&v"(kr[2]), "=&v"(kr[3]), "=&v"(kr[4]), "=&v"(kr[5]), "=&v"(kr[6]),
          "=&v"(kr[7])
        : "v"(kaddr[0]), "v"(kaddr[1]), "v"(kaddr[2]), "v"(kaddr[3])
        : "memory");
  }
}

// V^T operands of one tile for O^T = V^T P^T through transposing reads:
// vr[(ks MT + mt) 2 + u] holds dims 32 mt + .., keys 16 ks + 8 u + ..
template <int D>
__device__ __forceinline__ void read_v_tile(const uint32_t (&vaddr)[D / 32], u32x2_t (&vr)[D / 4]) {
  if constexpr (D == 128) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %32\n ds_read_b64_tr_b16 %1, %32 offset:2048\n"
        "ds_read_b64_tr_b16 %2, %33\n ds_read_b64_tr_b16 %3, %33 offset:2048\n"
        "ds_read_b64_tr_b16 %4, %34\n ds_read_b64_tr_b16 %5, %34 offset:2048\n"
        "ds_read_b64_tr_b16 %6, %35\n ds_read_b64_tr_b16 %7, %35 offset:2048\n"
        "ds_read_b64_tr_b16 %8, %32 offset:4096\n ds_read_b64_tr_b16 %9, %32 offset:6144\n"
        "ds_read_b64_tr_b16 %10, %33 offset:4096\n ds_read_b64_tr_b16 %11, %33 offset:6144\n"
        "ds_read_b64_tr_b16 %12, %34 offset:4096\n ds_read_b64_tr_b16 %13, %34 offset:6144\n"
        "ds_read_b64_tr_b16 %14, %35 offset:4096\n ds_read_b64_tr_b16 %15, %35 offset:6144\n"
        "ds_read_b64_tr_b16 %16, %32 offset:8192\n ds_read_b64_tr_b16 %17, %32 offset:10240\n"
        "ds_read_b64_tr_b16 %18, %33 offset:8192\n ds_read_b64_tr_b16 %19, %33 offset:10240\n"
        "ds_read_b64_tr_b16 %20, %34 offset:8192\n ds_read_b64_tr_b16 %21, %34 offset:10240\n"
        "ds_read_b64_tr_b16 %22, %35 offset:8192\n ds_read_b64_tr_b16 %23, %35 offset:10240\n"
        "ds_read_b64_tr_b16 %24, %32 offset:12288\n ds_read_b64_tr_b16 %25, %32 offset:14336\n"
        "ds_read_b64_tr_b16 %26, %33 offset:12288\n ds_read_b64_tr_b16 %27, %33 offset:14336\n"
        "ds_read_b64_tr_b16 %28, %34 offset:12288\n ds_read_b64_tr_b16 %29, %34 offset:14336\n"
        "ds_read_b64_tr_b16 %30, %35 offset:12288\n ds_read_b64_tr_b16 %31, %35 offset:14336\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(vr[0]), "=&v"(vr[1]), "=&v"(vr[2]), "=&v"(vr[3]), "=&v"(vr[4]), "=&v"(vr[5]), "=&v"(vr[6]),
          "=&v"(vr[7]), "=&v"(vr[8]), "=&v"(vr[9]), "=&v"(vr[10]), "=&v"(vr[11]), "=&v"(vr[12]), "=&v"(vr[13]),
          "=&v"(vr[14]), "=&v"(vr[15]), "=&v"(vr[16]), "=&v"(vr[17]), "=&v"(vr[18]), "=&v"(vr[19]),
          "=&v"(vr[20]), "=&v"(vr[21]), "=&v"(vr[22]), "=&v"(vr[23]), "=&v"(vr[24]), "=&v"(vr[25]),
          "=&v"(vr[26]), "=&v"(vr[27]), "=&v"(vr[28]), "=&v"(vr[29]), "=&v"(vr[30]), "=&v"(vr[31])
        : "v"(vaddr[0]), "v"(vaddr[1]), "v"(vaddr[2]), "v"(vaddr[3])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n ds_read_b64_tr_b16 %1, %16 offset:1024\n"
        "ds_read_b64_tr_b16 %2, %17\n ds_read_b64_tr_b16 %3, %17 offset:1024\n"
        "ds_read_b64_tr_b16 %4, %16 offset:2048\n ds_read_b64_tr_b16 %5, %16 offset:3072\n"
        "ds_read_b64_tr_b16 %6, %17 offset:2048\n ds_read_b64_tr_b16 %7, %17 offset:3072\n"
        "ds_read_b64_tr_b16 %8, %16 offset:4096\n ds_read_b64_tr_b16 %9, %16 offset:5120\n"
        "ds_read_b64_tr_b16 %10, %17 offset:4096\n ds_read_b64_tr_b16 %11, %17 offset:5120\n"
        "ds_read_b64_tr_b16 %12, %16 offset:6144\n ds_read_b64_tr_b16 %13, %16 offset:7168\n"
        "ds_read_b64_tr_b16 %14, %17 offset:6144\n ds_read_b64_tr_b16 %15, %17 offset:7168\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(vr[0]), "=&v"(vr[1]), "=&v"(vr[2]), "=&v"(vr[3]), "=&v"(vr[4]), "=&v"(vr[5]), "=&v"(vr[6]),
          "=&v"(vr[7]), "=&v"(vr[8]), "=&v"(vr[9]), "=&v"(vr[10]), "=&v"(vr[11]), "=&v"(vr[12]), "=&v"(vr[13]),
          "=&v"(vr[14]), "=&v"(vr[15])
        : "v"(vaddr[0]), "v"(vaddr[1])
        : "memory");
  }
}

// The same operand reads in two halves, so that other work can be issued
// while they are in flight: *_issue starts the LDS reads and *_wait waits for
// them. Between the two, only instructions that neither read nor write the
// destination registers may run (the tile copies of the persistent kernel).
// The wait takes every destination as an in-out operand, which keeps the
// registers in place and keeps the compiler from reading them before it.
template <int D>
__device__ __forceinline__ void read_k_issue(const uint32_t (&kaddr)[D / 16], u32x4_t (&kr)[D / 8]) {
  if constexpr (D == 128) {
    asm volatile(
        "ds_read_b128 %0, %16\n ds_read_b128 %1, %16 offset:8192\n"
        "ds_read_b128 %2, %17\n ds_read_b128 %3, %17 offset:8192\n"
        "ds_read_b128 %4, %18\n ds_read_b128 %5, %18 offset:8192\n"
        "ds_read_b128 %6, %19\n ds_read_b128 %7, %19 offset:8192\n"
        "ds_read_b128 %8, %20\n ds_read_b128 %9, %20 offset:8192\n"
        "ds_read_b128 %10, %21\n ds_read_b128 %11, %21 offset:8192\n"
        "ds_read_b128 %12, %22\n ds_read_b128 %13, %22 offset:8192\n"
        "ds_read_b128 %14, %23\n ds_read_b128 %15, %23 offset:8192"
        : "=&v"(kr[0]), "=&v"(kr[1]), "=&v"(kr[2]), "=&v"(kr[3]), "=&v"(kr[4]), "=&v"(kr[5]), "=&v"(kr[6]),
          "=&v"(kr[7]), "=&v"(kr[8]), "=&v"(kr[9]), "=&v"(kr[10]), "=&v"(kr[11]), "=&v"(kr[12]), "=&v"(kr[13]),
          "=&v"(kr[14]), "=&v"(kr[15])
        : "v"(kaddr[0]), "v"(kaddr[1]), "v"(kaddr[2]), "v"(kaddr[3]), "v"(kaddr[4]), "v"(kaddr[5]),
          "v"(kaddr[6]), "v"(kaddr[7])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %8\n ds_read_b128 %1, %8 offset:4096\n"
        "ds_read_b128 %2, %9\n ds_read_b128 %3, %9 offset:4096\n"
        "ds_read_b128 %4, %10\n ds_read_b128 %5, %10 offset:4096\n"
        "ds_read_b128 %6, %11\n ds_read_b128 %7, %11 offset:4096"
        : "=&v"(kr[0]), "=&v"(kr[1]), "=&v"(kr[2]), "=&v"(kr[3]), "=&v"(kr[4]), "=&v"(kr[5]), "=&v"(kr[6]),
          "=&v"(kr[7])
        : "v"(kaddr[0]), "v"(kaddr[1]), "v"(kaddr[2]), "v"(kaddr[3])
        : "memory");
  }
}

template <int D>
__device__ __forceinline__ void read_k_wait(u32x4_t (&kr)[D / 8]) {
  if constexpr (D == 128) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(kr[0]), "+v"(kr[1]), "+v"(kr[2]), "+v"(kr[3]), "+v"(kr[4]), "+v"(kr[5]), "+v"(kr[6]),
                   "+v"(kr[7]), "+v"(kr[8]), "+v"(kr[9]), "+v"(kr[10]), "+v"(kr[11]), "+v"(kr[12]),
                   "+v"(kr[13]), "+v"(kr[14]), "+v"(kr[15])
                 :
                 : "memory");
  } else {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(kr[0]), "+v"(kr[1]), "+v"(kr[2]), "+v"(kr[3]), "+v"(kr[4]), "+v"(kr[5]), "+v"(kr[6]),
                   "+v"(kr[7])
                 :
                 : "memory");
  }
}

template <int D>
__device__ __forceinline__ void read_v_issue(const uint32_t (&vaddr)[D / 32], u32x2_t (&vr)[D / 4]) {
  if constexpr (D == 128) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %32\n ds_read_b64_tr_b16 %1, %32 offset:2048\n"
        "ds_read_b64_tr_b16 %2, %33\n ds_read_b64_tr_b16 %3, %33 offset:2048\n"
        "ds_read_b64_tr_b16 %4, %34\n ds_read_b64_tr_b16 %5, %34 offset:2048\n"
        "ds_read_b64_tr_b16 %6, %35\n ds_read_b64_tr_b16 %7, %35 offset:2048\n"
        "ds_read_b64_tr_b16 %8, %32 offset:4096\n ds_read_b64_tr_b16 %9, %32 offset:6144\n"
        "ds_read_b64_tr_b16 %10, %33 offset:4096\n ds_read_b64_tr_b16 %11, %33 offset:6144\n"
        "ds_read_b64_tr_b16 %12, %34 offset:4096\n ds_read_b64_tr_b16 %13, %34 offset:6144\n"
        "ds_read_b64_tr_b16 %14, %35 offset:4096\n ds_read_b64_tr_b16 %15, %35 offset:6144\n"
        "ds_read_b64_tr_b16 %16, %32 offset:8192\n ds_read_b64_tr_b16 %17, %32 offset:10240\n"
        "ds_read_b64_tr_b16 %18, %33 offset:8192\n ds_read_b64_tr_b16 %19, %33 offset:10240\n"
        "ds_read_b64_tr_b16 %20, %34 offset:8192\n ds_read_b64_tr_b16 %21, %34 offset:10240\n"
        "ds_read_b64_tr_b16 %22, %35 offset:8192\n ds_read_b64_tr_b16 %23, %35 offset:10240\n"
        "ds_read_b64_tr_b16 %24, %32 offset:12288\n ds_read_b64_tr_b16 %25, %32 offset:14336\n"
        "ds_read_b64_tr_b16 %26, %33 offset:12288\n ds_read_b64_tr_b16 %27, %33 offset:14336\n"
        "ds_read_b64_tr_b16 %28, %34 offset:12288\n ds_read_b64_tr_b16 %29, %34 offset:14336\n"
        "ds_read_b64_tr_b16 %30, %35 offset:12288\n ds_read_b64_tr_b16 %31, %35 offset:14336"
        : "=&v"(vr[0]), "=&v"(vr[1]), "=&v"(vr[2]), "=&v"(vr[3]), "=&v"(vr[4]), "=&v"(vr[5]), "=&v"(vr[6]),
          "=&v"(vr[7]), "=&v"(vr[8]), "=&v"(vr[9]), "=&v"(vr[10]), "=&v"(vr[11]), "=&v"(vr[12]), "=&v"(vr[13]),
          "=&v"(vr[14]), "=&v"(vr[15]), "=&v"(vr[16]), "=&v"(vr[17]), "=&v"(vr[18]), "=&v"(vr[19]),
          "=&v"(vr[20]), "=&v"(vr[21]), "=&v"(vr[22]), "=&v"(vr[23]), "=&v"(vr[24]), "=&v"(vr[25]),
          "=&v"(vr[26]), "=&v"(vr[27]), "=&v"(vr[28]), "=&v"(vr[29]), "=&v"(vr[30]), "=&v"(vr[31])
        : "v"(vaddr[0]), "v"(vaddr[1]), "v"(vaddr[2]), "v"(vaddr[3])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n ds_read_b64_tr_b16 %1, %16 offset:1024\n"
        "ds_read_b64_tr_b16 %2, %17\n ds_read_b64_tr_b16 %3, %17 offset:1024\n"
        "ds_read_b64_tr_b16 %4, %16 offset:2048\n ds_read_b64_tr_b16 %5, %16 offset:3072\n"
        "ds_read_b64_tr_b16 %6, %17 offset:2048\n ds_read_b64_tr_b16 %7, %17 offset:3072\n"
        "ds_read_b64_tr_b16 %8, %16 offset:4096\n ds_read_b64_tr_b16 %9, %16 offset:5120\n"
        "ds_read_b64_tr_b16 %10, %17 offset:4096\n ds_read_b64_tr_b16 %11, %17 offset:5120\n"
        "ds_read_b64_tr_b16 %12, %16 offset:6144\n ds_read_b64_tr_b16 %13, %16 offset:7168\n"
        "ds_read_b64_tr_b16 %14, %17 offset:6144\n ds_read_b64_tr_b16 %15, %17 offset:7168"
        : "=&v"(vr[0]), "=&v"(vr[1]), "=&v"(vr[2]), "=&v"(vr[3]), "=&v"(vr[4]), "=&v"(vr[5]), "=&v"(vr[6]),
          "=&v"(vr[7]), "=&v"(vr[8]), "=&v"(vr[9]), "=&v"(vr[10]), "=&v"(vr[11]), "=&v"(vr[12]), "=&v"(vr[13]),
          "=&v"(vr[14]), "=&v"(vr[15])
        : "v"(vaddr[0]), "v"(vaddr[1])
        : "memory");
  }
}

template <int D>
__device__ __forceinline__ void read_v_wait(u32x2_t (&vr)[D / 4]) {
  if constexpr (D == 128) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(vr[0]), "+v"(vr[1]), "+v"(vr[2]), "+v"(vr[3]), "+v"(vr[4]), "+v"(vr[5]), "+v"(vr[6]),
                   "+v"(vr[7]), "+v"(vr[8]), "+v"(vr[9]), "+v"(vr[10]), "+v"(vr[11]), "+v"(vr[12]),
                   "+v"(vr[13]), "+v"(vr[14]), "+v"(vr[15]), "+v"(vr[16]), "+v"(vr[17]), "+v"(vr[18]),
                   "+v"(vr[19]), "+v"(vr[20]), "+v"(vr[21]), "+v"(vr[22]), "+v"(vr[23]), "+v"(vr[24]),
                   "+v"(vr[25]), "+v"(vr[26]), "+v"(vr[27]), "+v"(vr[28]), "+v"(vr[29]), "+v"(vr[30]),
                   "+v"(vr[31])
                 :
                 : "memory");
  } else {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(vr[0]), "+v"(vr[1]), "+v"(vr[2]), "+v"(vr[3]), "+v"(vr[4]), "+v"(vr[5]), "+v"(vr[6]),
                   "+v"(vr[7]), "+v"(vr[8]), "+v"(vr[9]), "+v"(vr[10]), "+v"(vr[11]), "+v"(vr[12]),
                   "+v"(vr[13]), "+v"(vr[14]), "+v"(vr[15])
                 :
                 : "memory");
  }
}

// s_waitcnt vmcnt(N) for any N < 64 (expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm_le() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xf00 | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(n) for a count known only at run time: the counts the
// kernels use have their own instruction; any other count waits for every
// operation in flight, which is always safe
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 1: wait_vm_le<1>(); break;
    case 4: wait_vm_le<4>(); break;
    case 5: wait_vm_le<5>(); break;
    case 8: wait_vm_le<8>(); break;
    case 9: wait_vm_le<9>(); break;
    case 12: wait_vm_le<12>(); break;
    case 16: wait_vm_le<16>(); break;
    default: wait_vm_le<0>(); break;
  }
}

// s_waitcnt vmcnt(n) for 0 <= n: counts up to 15 have their own instruction,
// larger ones wait until 15 remain (more than needed, always safe)
__device__ __forceinline__ void wait_vm_upto(int n) {
  switch (n) {
    case 0: wait_vm_le<0>(); break;
    case 1: wait_vm_le<1>(); break;
    case 2: wait_vm_le<2>(); break;
    case 3: wait_vm_le<3>(); break;
    case 4: wait_vm_le<4>(); break;
    case 5: wait_vm_le<5>(); break;
    case 6: wait_vm_le<6>(); break;
    case 7: wait_vm_le<7>(); break;
    case 8: wait_vm_le<8>(); break;
    case 9: wait_vm_le<9>(); break;
    case 10: wait_vm_le<10>(); break;
    case 11: wait_vm_le<11>(); break;
    case 12: wait_vm_le<12>(); break;
    case 13: wait_vm_le<13>(); break;
    case 14: wait_vm_le<14>(); break;
    default: wait_vm_le<15>(); break;
  }
}

}  // namespace seer
