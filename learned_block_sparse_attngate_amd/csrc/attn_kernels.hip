// Causal GQA block-sparse / dense FlashAttention-style forward for gfx950,
// plus the dense variant that records per-tile row maxima for the
// 2D-maxpooled ground truth.
//
// Method ("SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs",
// explainer section 3.4): the attention map is cut into 64 x 64 tiles aligned
// with the gate's blocks; a tile whose block-mask entry is 0 is skipped whole
// (no QK^T, no softmax, no PV and no K/V loads), a tile whose entry is 1 is
// processed with the FlashAttention-2 online softmax. For the ground truth
// (same page, "Training Procedure", customized training kernel) the kernel
// stores r = rowmax(S_ij) per query row and key tile, and after the row is
// finished rescales it with the final statistics (exp(r - m) / l) and takes a
// column max over the query block.
//
// Design for CDNA4:
//  * one workgroup = one (batch, query head, query block) row = 64 queries,
//    2 wavefronts x 32 queries, two workgroups per SIMD so that one wave's
//    MFMA work overlaps the other's softmax; Q stays in registers;
//  * both contractions use v_mfma_f32_32x32x16_bf16 with the matrix roles
//    chosen so the softmax is lane-local: S^T = K Q^T puts one query per lane
//    (32 of its keys in the lane, the other 32 in lane l^32), and
//    O^T = V^T P^T consumes the S^T registers directly as the B operand, so P
//    never goes through LDS;
//  * K and V tiles move HBM -> LDS with buffer_load_dwordx4 ... lds (no
//    register staging); the XOR swizzle is applied on the source side so the
//    LDS image is conflict-free for the 16-byte K operand reads and for the
//    ds_read_b64_tr_b16 transposing reads that build the V^T operand;
//  * K and V have one LDS buffer each and are refilled independently: the K
//    copy of the next tile starts as soon as both waves hold this tile's K
//    operands, the V copy as soon as they hold its V operands, so each copy
//    overlaps roughly one full tile of work. The operand reads are
//    inline-assembly blocks that wait for their own results before they end;
//    this keeps the compiler from inserting a wait for every copy in flight
//    before each LDS read, and the copies are tracked with explicit vmcnt
//    waits instead;
//  * the active key blocks of a row are compacted on chip from the mask row
//    into an LDS list (ascending), so masked tiles cost neither time nor HBM
//    traffic and no separate compaction launch is needed; the diagonal tile's
//    copy is started before the compaction;
//  * the workgroup order keeps one KV group's K/V hot at a time and launches
//    the heaviest rows first;
//  * block-sparse rows longer than 1024 blocks are cut into key chunks of 512
//    blocks: a work item is (row, chunk), items go chunk by chunk, so all XCDs
//    read one chunk of one KV group's K/V at a time; an item writes its
//    normalized fp32 partial and log-sum-exp to the workspace and a second
//    kernel merges the chunks of each row (split-KV); each item walks its
//    tiles in a circular order phased by its dispatch slot, so the items
//    resident on an XCD read neighbouring key blocks at the same time.
#include <stdlib.h>

#include <type_traits>

#include "seer_device.h"
#include "seer_internal.h"

namespace seer {

namespace {

constexpr int kThreads = 128;            // 2 wavefronts
constexpr int kListCap = 2048;           // mask columns compacted per pass
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleSlack = 8.0f;    // log2 units the running max may lag by
constexpr int kBufferWord3 = 0x00020000; // gfx9-family raw buffer resource, dword 3
constexpr int kXcds = 8;                 // workgroups are dealt round-robin to the 8 XCDs
constexpr int kSweepPhases = 128;        // resident workgroups per XCD (32 CUs x 4)

enum Mode { kSparse = 0, kDense = 1, kDenseGt = 2 };

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

// s_waitcnt vmcnt(n) (expcnt and lgkmcnt left at their maxima)
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0f70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0f71); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0f74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0f75); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0f78); break;
    default: __builtin_amdgcn_s_waitcnt(0x0f79); break;
  }
}

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

template <int D, int MODE>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(AttnArgs p) {
  constexpr int CPR = D / 8;               // 16-byte chunks per K/V row
  constexpr int KS = D / 16;               // MFMA k-steps for S^T
  constexpr int MT = D / 32;               // MFMA m-tiles for O^T
  constexpr int RPI = 64 / CPR;            // tile rows per copy instruction
  constexpr int NDMA = 32 / RPI;           // copy instructions per wave per operand (32 rows)

  __shared__ uint4 Ks[kBlock * CPR];       // K tile [64 keys][D], swizzled chunks
  __shared__ uint4 Vs[kBlock * CPR];       // V tile [64 keys][D], swizzled chunks
  __shared__ uint16_t list[MODE == kSparse ? kListCap : 1];
  __shared__ int wsum[2];
  __shared__ float lse_s[MODE == kDenseGt ? kBlock : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // ---- which row ---------------------------------------------------------
  // Workgroups are dispatched round-robin over the 8 XCDs (each with its own
  // L2); all orders below launch the heaviest rows (last query blocks) first.
  //  0: heads interleaved, all KV groups at once;
  //  1: the query heads of one KV group on one XCD;
  //  2: KV-group major: every XCD works on the same KV group at a time, so
  //     the K/V working set is one group;
  //  3: KV-group major, then head major inside the group.
  const int BH = p.B * p.Hq;
  const int w = blockIdx.x;
  int qb, bh;
  int chunk = 0;                                  // block-sparse: key chunk of this work item
  if constexpr (MODE == kSparse) {
    // Key-chunked items: (batch, KV group) major, then chunk c ascending, then
    // head, then query block descending. Consecutive items go round-robin over
    // the XCDs, so all of them work on one C-block K/V chunk of one group at a
    // time and that chunk stays in each XCD's L2.
    const int gi = static_cast<int>(w / p.items_per_group);
    long long r = w - gi * p.items_per_group;
    int c = 0;
    while (true) {
      const long long n = static_cast<long long>(p.group) * (p.nb - c * p.chunk);   // items of chunk c
      if (r < n) break;
      r -= n;
      ++c;
    }
    const int rows = p.nb - c * p.chunk;            // query blocks qb >= c*C
    const int hig = static_cast<int>(r / rows);
    qb = p.nb - 1 - static_cast<int>(r % rows);
    chunk = c;
    const int bb = gi / p.Hkv, gg = gi - bb * p.Hkv;
    bh = bb * p.Hq + gg * p.group + hig;
  } else if (p.sched >= 2) {
    const int R = p.group * p.nb;                 // rows per (batch, KV group)
    const int gi = w / R, r = w - gi * R;         // gi = b * Hkv + g
    int hig;
    if (p.sched == 2) { qb = p.nb - 1 - r / p.group; hig = r % p.group; }
    else { hig = r / p.nb; qb = p.nb - 1 - r % p.nb; }
    const int bb = gi / p.Hkv, gg = gi - bb * p.Hkv;
    bh = bb * p.Hq + gg * p.group + hig;
  } else {
    qb = p.nb - 1 - w / BH;
    int local = w % BH;
    if (p.sched == 1) local = (local & 7) * (BH >> 3) + (local >> 3);
    bh = local;
  }
  const int b = bh / p.Hq;
  const int h = bh - b * p.Hq;
  const int g = h / p.group;
  const size_t kv_off = (static_cast<size_t>(b) * p.Hkv + g) * p.hs * D;
  const uint16_t* __restrict__ Kg = p.k + kv_off;
  const uint16_t* __restrict__ Vg = p.v + kv_off;

  // ---- HBM -> LDS copies ---------------------------------------------------
  // Instruction i, lane l writes LDS bytes [1024 i + 16 l) of this wave's half
  // (rows 32w .. 32w+31): tile row r = 32w + RPI*i + l/CPR, physical chunk
  // l%CPR, holding logical chunk (l%CPR) ^ swz(r). With the swizzles above the
  // V chunk does not depend on i and the K chunk takes four values, so a few
  // per-lane byte offsets address every instruction. The buffer resource starts
  // at the tile and ends at the head's last row, so rows past the sequence
  // (ragged last tile) read as zeros: their scores are masked by causality and
  // their P is 0.
  uint32_t kofs[4], vofs;
  {
    const int r0 = 32 * wave + lane / CPR;
    const int pc = lane % CPR;
#pragma unroll
    for (int v = 0; v < 4; ++v) kofs[v] = static_cast<uint32_t>(r0 * 2 * D + 16 * (pc ^ swz_k<D>(r0 + RPI * v)));
    vofs = static_cast<uint32_t>(r0 * 2 * D + 16 * (pc ^ swz_v<D>(r0)));
  }
  auto issue_k = [&](int kb) {
    const int key0 = kb * kBlock;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Kg + static_cast<size_t>(key0) * D), 0,
                                                      (p.S - key0) * 2 * D, kBufferWord3);
    char* dst = reinterpret_cast<char*>(Ks) + 32 * wave * D * 2;
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const uint32_t ko = (D == 128 ? kofs[i & 3] : kofs[0]) + static_cast<uint32_t>(RPI * i * 2 * D);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + 1024 * i), 16, ko, 0, 0, 0);
    }
  };
  auto issue_v = [&](int kb) {
    const int key0 = kb * kBlock;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Vg + static_cast<size_t>(key0) * D), 0,
                                                      (p.S - key0) * 2 * D, kBufferWord3);
    char* dst = reinterpret_cast<char*>(Vs) + 32 * wave * D * 2;
#pragma unroll
    for (int i = 0; i < NDMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + 1024 * i), 16,
                                               vofs + static_cast<uint32_t>(RPI * i * 2 * D), 0, 0, 0);
  };

  // LDS byte addresses of the operand reads (loop invariant)
  uint32_t kaddr[KS], vaddr[MT];
  {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kaddr[ks] = lds_addr(Ks) + l32 * 2 * D + 16 * ((2 * ks + hl) ^ swz_k<D>(l32));
    // transposing reads: within each 16-lane group, lane 4j+a points at 4
    // dims of key j; the instruction hands lane i the 4 keys of dim i
    const int G = lane >> 4, j = (lane >> 2) & 3, a = lane & 3;
    const int key = 4 * (G >> 1) + j;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      vaddr[mt] = lds_addr(Vs) + key * 2 * D + 16 * ((4 * mt + 2 * (G & 1) + (a >> 1)) ^ swz_v<D>(key)) + 8 * (a & 1);
  }

  // the diagonal tile is processed first; start its copy before anything else
  // (in block-sparse mode only the item whose chunk holds the diagonal has it)
  if (MODE != kSparse || qb < (chunk + 1) * p.chunk) {
    issue_k(qb);
    issue_v(qb);
  }

  // ---- Q fragment (B operand of S^T = K Q^T), resident for the row ------
  const int q_local = wave * 32 + l32;            // query row within the block
  const int t = qb * kBlock + q_local;            // query position
  const bool t_ok = t < p.S;
  uint4 qreg[KS];
  {
    const uint16_t* qrow = p.q + (static_cast<size_t>(bh) * p.hs + (t_ok ? t : 0)) * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[ks] = t_ok ? *reinterpret_cast<const uint4*>(qrow + 16 * ks) : make_uint4(0, 0, 0, 0);
  }

  const float c = p.scale_log2;                   // log2(e) / sqrt(D)
  float m = -INFINITY;                            // running max (log2 units, may lag by kRescaleSlack)
  float lsum = 0.f;                               // this lane's partial row sum
  f32x16_t oacc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) oacc[i] = f32x16_t{};

  const long long ntri_off = static_cast<long long>(qb) * (qb + 1) / 2;  // ground-truth scratch offset of this row

  // One tile. On entry the copies of tile kb are in flight or landed, K issued
  // before V. `first`: nothing but this tile's V copy was issued after its K
  // copy. `stores_pending`: ground-truth stores issued after the last V copy.
  int stores_pending = 0;
  auto compute = [&](auto diag_tag, int kb, int next, bool first) {
    constexpr bool kDiag = decltype(diag_tag)::value;   // the diagonal tile needs element causality
    // ---- K: wait for the copy (only V of this tile and newer stores may be outstanding)
    wait_vmcnt(first ? NDMA : NDMA + stores_pending);
    wg_barrier();
    u32x4_t kr[2 * KS];                           // kr[2 ks + mt]: keys 32 mt + l32, dims 16 ks + 8 hl ..
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
    wg_barrier();                                  // both waves hold K: refill the K buffer
    if (next >= 0) issue_k(next);

    // ---- S^T = K Q^T (32 keys x 32 queries per m-tile, two m-tiles)
    f32x16_t sacc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        sacc[mt] = mfma_32x32x16(__builtin_bit_cast(uint4, kr[2 * ks + mt]), qreg[ks], sacc[mt]);

    // element causality on the diagonal tile; row max
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (kDiag) {
          const int key = 32 * mt + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (key > q_local) sacc[mt][r] = -INFINITY;
        }
        mx = fmaxf(mx, sacc[mt][r]);
      }
    }
    mx = pair_max(mx) * c;                         // row max of this tile, log2 units
    int stores_now = 0;
    if constexpr (MODE == kDenseGt) {
      if (hl == 0) p.rmax[((static_cast<size_t>(bh) * p.ntri + ntri_off + kb) << 6) + q_local] = mx;
      stores_now = 1;
    }

    // ---- V: wait for the copy (the K copy of `next` and this tile's store may be newer)
    wait_vmcnt((next >= 0 ? NDMA : 0) + stores_now);
    wg_barrier();
    u32x2_t vr[8 * MT];                            // vr[(ks MT + mt) 2 + u]: dims 32 mt + .., keys 16 ks + 8 u + ..
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
    wg_barrier();                                  // both waves hold V: refill the V buffer
    if (next >= 0) issue_v(next);
    stores_pending = stores_now;

    // lazy rescale: move the running max only when it grows by > slack
    const bool upd = mx > m + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(upd)) {
      const float mn = upd ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mn);   // m = -inf on the first tile: alpha = 0
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < MT; ++i) oacc[i] *= alpha;
      m = mn;
    }
    // P = exp2(s*c - m), packed to bf16 in the B-operand layout of O^T = V^T P^T
    uint4 pb[4];
    float ls = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float e[8];
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
          e[s8] = __builtin_amdgcn_exp2f(fmaf(sacc[mt][8 * hh + s8], c, -m));
          ls += e[s8];
        }
        pb[2 * mt + hh] = make_uint4(pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]),
                                     pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7]));
      }
    }
    lsum += ls;
    // ---- O^T += V^T P^T (32 dims x 32 queries per m-tile, 4 k-steps of 16 keys)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x2_t lo = vr[(ks * MT + mt) * 2], hi = vr[(ks * MT + mt) * 2 + 1];
        oacc[mt] = mfma_32x32x16(make_uint4(lo.x, lo.y, hi.x, hi.y), pb[ks], oacc[mt]);
      }
  };

  // ---- main loop over active key blocks -----------------------------------
  // The diagonal block (the only one needing element causality) goes first,
  // then the other active blocks: in block-sparse mode in the circular order
  // below, in dense mode ascending.
  if constexpr (MODE == kSparse) {
    const uint8_t* mrow = p.mask + (static_cast<size_t>(bh) * p.nb + qb) * p.nb;
    const int c0 = chunk * p.chunk;                     // this item's key blocks: [c0, c1) plus maybe the diagonal
    const int c1 = min(qb, c0 + p.chunk);               // off-diagonal candidates (C <= kListCap)
    const bool has_diag = qb < c0 + p.chunk;
    const uint32_t list_lds = lds_addr(list), wsum_lds = lds_addr(wsum);
    // mask bytes of columns [c0, c1) -> 16 flags per thread
    uint32_t bits = 0;
    {
      const int j0 = c0 + 16 * tid;
      if (j0 < c1) {
        if (j0 + 16 <= c1 && ((reinterpret_cast<uintptr_t>(mrow + j0) & 15) == 0)) {
          const uint4 v4 = *reinterpret_cast<const uint4*>(mrow + j0);
          const uint32_t wv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if ((wv[e >> 2] >> (8 * (e & 3))) & 0xffu) bits |= 1u << e;
        } else {
          for (int e = 0; e < 16 && j0 + e < c1; ++e)
            if (mrow[j0 + e]) bits |= 1u << e;
        }
      }
    }
    const bool diag_on = has_diag && __builtin_amdgcn_readfirstlane(static_cast<int>(mrow[qb])) != 0;
    // ascending list of the active columns. Only fence-free barriers and LDS
    // reads outside the compiler's tracking here: the diagonal tile's copy may
    // be in flight.
    int cnt;
    {
      const int nset = __builtin_popcount(bits);
      const int inc = wave_inclusive_scan(nset, lane);
      if (lane == kWave - 1) wsum[wave] = inc;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      wg_barrier();
      const int w0 = static_cast<int>(lds_read_u32(wsum_lds));
      cnt = __builtin_amdgcn_readfirstlane(w0 + static_cast<int>(lds_read_u32(wsum_lds + 4)));
      int pos = inc - nset + (wave == 1 ? w0 : 0);
      const int j0 = c0 + 16 * tid;
      while (bits) {
        const int e = __builtin_ctz(bits);
        bits &= bits - 1;
        list[pos++] = static_cast<uint16_t>(j0 + e);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      wg_barrier();
    }
    // Circular sweep: the list is walked starting at a position proportional
    // to this workgroup's place in its XCD's dispatch sequence (one phase per
    // resident slot) and wraps around. Workgroups of one XCD start one after
    // another and walk the same key range at about the same speed, so the
    // ones resident together read neighbouring key blocks at any moment and
    // the XCD's L2 holds a narrow window of K/V instead of the whole range.
    const int rot = p.rotate ? static_cast<int>((static_cast<unsigned>((w / kXcds) % kSweepPhases) *
                                                 static_cast<unsigned>(cnt)) / kSweepPhases)
                             : 0;
    auto entry = [&](int n) {                   // n-th tile of the sweep
      const int i = rot + n < cnt ? rot + n : rot + n - cnt;
      return __builtin_amdgcn_readfirstlane(static_cast<int>(lds_read_u16(list_lds + 2 * i)));
    };
    bool issued = false;                        // the sweep's first tile already in flight
    if (diag_on) {
      const int nxt = cnt > 0 ? entry(0) : -1;
      compute(std::true_type{}, qb, nxt, true);
      issued = cnt > 0;
    } else if (has_diag) {
      wait_vmcnt(0);                            // the early copy of the diagonal tile is not used
      wg_barrier();
    }
    if (cnt > 0) {
      int kb = entry(0);
      bool first = !issued;
      if (!issued) { issue_k(kb); issue_v(kb); }
      for (int n = 0; n < cnt; ++n) {
        const int next = n + 1 < cnt ? entry(n + 1) : -1;
        compute(std::false_type{}, kb, next, first);
        first = false;
        kb = next;
      }
    }
  } else {
    compute(std::true_type{}, qb, qb > 0 ? 0 : -1, true);
    for (int kb = 0; kb < qb; ++kb) compute(std::false_type{}, kb, kb + 1 < qb ? kb + 1 : -1, false);
  }

  // ---- epilogue: normalize, store O and LSE --------------------------------
  const float ltot = pair_sum(lsum);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  const float lse2 = ltot > 0.f ? m + __log2f(ltot) : -INFINITY;
  if constexpr (MODE == kSparse) {
    if (qb >= p.chunk) {
      // row spans several chunks: normalized fp32 partial + its log2-sum-exp
      float* po = p.part_o + (static_cast<size_t>(w) * kBlock + q_local) * D;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *reinterpret_cast<float4*>(po + 32 * mt + 8 * r4 + 4 * hl) =
              make_float4(oacc[mt][4 * r4] * inv, oacc[mt][4 * r4 + 1] * inv, oacc[mt][4 * r4 + 2] * inv,
                          oacc[mt][4 * r4 + 3] * inv);
      if (hl == 0) p.part_l[static_cast<size_t>(w) * kBlock + q_local] = lse2;
      return;
    }
  }
  if (t_ok) {
    const size_t obase = (static_cast<size_t>(bh) * p.hs + t) * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dim = 32 * mt + 8 * r4 + 4 * hl;
        const float o0 = oacc[mt][4 * r4 + 0] * inv, o1 = oacc[mt][4 * r4 + 1] * inv;
        const float o2 = oacc[mt][4 * r4 + 2] * inv, o3 = oacc[mt][4 * r4 + 3] * inv;
        if (p.out_bf16) {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + obase + dim) =
              make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(p.out) + obase + dim) = make_float4(o0, o1, o2, o3);
        }
      }
    }
    if (p.lse != nullptr && hl == 0) p.lse[static_cast<size_t>(bh) * p.hs + t] = lse2 * kLn2;
  }

  if constexpr (MODE == kDenseGt) {
    // gt[qb, kb] = max over the block's queries of exp2(r - lse2); 0 above the diagonal
    if (hl == 0) lse_s[q_local] = t_ok ? lse2 : INFINITY;
    __syncthreads();                              // lse_s and this row's r writes visible to the workgroup
    float* gtrow = p.gt + (static_cast<size_t>(bh) * p.nb + qb) * p.nb;
    for (int kb = tid; kb < p.nb; kb += kThreads) {
      float best = 0.f;
      if (kb <= qb) {
        const float4* rr = reinterpret_cast<const float4*>(
            p.rmax + ((static_cast<size_t>(bh) * p.ntri + ntri_off + kb) << 6));
#pragma unroll 4
        for (int q4 = 0; q4 < 16; ++q4) {
          const float4 v = rr[q4];
          best = fmaxf(best, exp2f(v.x - lse_s[4 * q4 + 0]));
          best = fmaxf(best, exp2f(v.y - lse_s[4 * q4 + 1]));
          best = fmaxf(best, exp2f(v.z - lse_s[4 * q4 + 2]));
          best = fmaxf(best, exp2f(v.w - lse_s[4 * q4 + 3]));
        }
      }
      gtrow[kb] = best;
    }
  }
}

// Merge the per-chunk partials of rows spanning several key chunks:
// O = sum_c w_c O_c / sum_c w_c, w_c = 2^(L_c - max L), LSE = max L + log2(sum w).
// One workgroup per such row; thread t handles query t/4, dims 32*(t%4) ...
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs p) {
  constexpr int DPT = D / 4;                    // dims per thread
  const int rows = p.nb - p.chunk;              // query blocks qb >= C per head
  const int bh = blockIdx.x / rows;
  const int qb = p.chunk + blockIdx.x % rows;
  const int b = bh / p.Hq, h = bh % p.Hq;
  const int g = h / p.group, hig = h % p.group;
  const long long gi = static_cast<long long>(b) * p.Hkv + g;
  const int q = threadIdx.x >> 2, d0 = (threadIdx.x & 3) * DPT;
  const int nchunks = qb / p.chunk + 1;
  auto item = [&](int c) {                      // work-item index of (row, chunk c)
    long long before = 0;
    for (int cc = 0; cc < c; ++cc) before += static_cast<long long>(p.group) * (p.nb - cc * p.chunk);
    const int rows_c = p.nb - c * p.chunk;
    return gi * p.items_per_group + before + static_cast<long long>(hig) * rows_c + (p.nb - 1 - qb);
  };
  float lmax = -INFINITY;
  for (int c = 0; c < nchunks; ++c) lmax = fmaxf(lmax, p.part_l[item(c) * kBlock + q]);
  float acc[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  if (lmax > -INFINITY) {
    for (int c = 0; c < nchunks; ++c) {
      const long long it = item(c);
      const float wc = __builtin_amdgcn_exp2f(p.part_l[it * kBlock + q] - lmax);
      wsum += wc;
      const float4* src = reinterpret_cast<const float4*>(p.part_o + (it * kBlock + q) * D + d0);
#pragma unroll
      for (int i = 0; i < DPT / 4; ++i) {
        const float4 v = src[i];
        acc[4 * i] = fmaf(wc, v.x, acc[4 * i]);
        acc[4 * i + 1] = fmaf(wc, v.y, acc[4 * i + 1]);
        acc[4 * i + 2] = fmaf(wc, v.z, acc[4 * i + 2]);
        acc[4 * i + 3] = fmaf(wc, v.w, acc[4 * i + 3]);
      }
    }
  }
  const int t = qb * kBlock + q;
  if (t >= p.S) return;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const size_t obase = (static_cast<size_t>(bh) * p.hs + t) * D + d0;
  if (p.out_bf16) {
    uint16_t* o = static_cast<uint16_t*>(p.out) + obase;
#pragma unroll
    for (int i = 0; i < DPT / 4; ++i)
      *reinterpret_cast<uint2*>(o + 4 * i) = make_uint2(pack_bf16x2(acc[4 * i] * inv, acc[4 * i + 1] * inv),
                                                        pack_bf16x2(acc[4 * i + 2] * inv, acc[4 * i + 3] * inv));
  } else {
    float* o = static_cast<float*>(p.out) + obase;
#pragma unroll
    for (int i = 0; i < DPT / 4; ++i)
      *reinterpret_cast<float4*>(o + 4 * i) =
          make_float4(acc[4 * i] * inv, acc[4 * i + 1] * inv, acc[4 * i + 2] * inv, acc[4 * i + 3] * inv);
  }
  if (p.lse != nullptr && d0 == 0)
    p.lse[static_cast<size_t>(bh) * p.hs + t] = wsum > 0.f ? (lmax + __log2f(wsum)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_d(const AttnArgs& a, int mode, hipStream_t st) {
  const dim3 block(kThreads);
  if (mode == kSparse) {
    const dim3 grid(static_cast<unsigned>(static_cast<long long>(a.B) * a.Hkv * a.items_per_group));
    hipLaunchKernelGGL((attn_fwd_kernel<D, kSparse>), grid, block, 0, st, a);
    if (a.nchunk > 1) {
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const dim3 cgrid(static_cast<unsigned>(a.B) * a.Hq * (a.nb - a.chunk));
      hipLaunchKernelGGL((attn_combine_kernel<D>), cgrid, dim3(256), 0, st, a);
    }
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>(a.B) * a.Hq * a.nb);
  if (mode == kDense) hipLaunchKernelGGL((attn_fwd_kernel<D, kDense>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((attn_fwd_kernel<D, kDenseGt>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

// Key blocks per chunk of the block-sparse work items. Up to 1024 blocks
// (64k tokens) a row is one item; longer rows are cut into chunks of 512
// blocks, which the XCDs sweep together. SEER_ATTN_CHUNK overrides the chunk
// (rounded to a multiple of 16, at most the on-chip list capacity).
int sparse_chunk_blocks(int nb) {
  static const int forced = [] {
    const char* v = getenv("SEER_ATTN_CHUNK");
    if (v == nullptr) return 0;
    int x = atoi(v);
    if (x < 16) x = 16;
    if (x > kListCap) x = kListCap;
    return x / 16 * 16;
  }();
  if (forced) return forced;
  return nb > 1024 ? 512 : kListCap;
}

// Circular sweep of each row's tiles (on by default; SEER_ATTN_ROTATE=0 turns
// it off). It changes only the order in which a row's tiles are accumulated.
int sparse_rotate(int nchunk) {
  (void)nchunk;
  static const int forced = [] {
    const char* v = getenv("SEER_ATTN_ROTATE");
    return v == nullptr ? -1 : (atoi(v) != 0);
  }();
  return forced >= 0 ? forced : 1;
}

long long sparse_items_per_group(int nb, int group, int chunk) {
  const long long nc = (nb + chunk - 1) / chunk;
  return static_cast<long long>(group) * (nc * nb - static_cast<long long>(chunk) * nc * (nc - 1) / 2);
}

size_t sparse_workspace_bytes(int B, int Hkv, int group, int nb, int D, int chunk) {
  if (nb <= chunk) return 0;
  const size_t items = static_cast<size_t>(B) * Hkv * sparse_items_per_group(nb, group, chunk);
  return items * kBlock * (static_cast<size_t>(D) + 1) * sizeof(float);
}

hipError_t launch_attn(const AttnArgs& a, int mode, hipStream_t st) {
  if (a.D == 64) return launch_d<64>(a, mode, st);
  return launch_d<128>(a, mode, st);
}

}  // namespace seer
