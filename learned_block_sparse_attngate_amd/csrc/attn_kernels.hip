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
#include "seer_device.h"
#include "seer_internal.h"
#include "tile_ops.h"

namespace seer {

namespace {

constexpr int kThreads = 128;            // 2 wavefronts
constexpr int kListCap = 2048;           // mask columns compacted per pass
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleSlack = 8.0f;    // log2 units the running max may lag by
constexpr int kXcds = 8;                 // workgroups are dealt round-robin to the 8 XCDs
// phases of the block-sparse circular sweep: twice the resident workgroups
// per XCD (32 CUs x 4); with 32/8 heads at 90% it measured 3% faster at 32k
// than 128 phases, 64, 512 and 1024 phases slower
constexpr int kSweepPhases = 256;

enum Mode {
  kSparse = 0,
  kDense = 1,
  kDenseGt = 2,
};

// Partial-output slots before query block qb of one head in the XCD-owned
// path: rows qb' >= C own qb'/C + 1 slots each (one per key chunk they reach;
// the diagonal chunk's slot is not written).
__device__ __host__ __forceinline__ long long xcd_slot_base(long long qb, long long C) {
  const long long k = qb / C;
  return qb + C * k * (k - 1) / 2 + k * (qb - k * C) - C;
}


// S^T = K Q^T for one tile (32 keys x 32 queries per m-tile, two m-tiles),
// element causality on the diagonal tile, and the row maximum of the tile in
// log2 units (c = log2(e) / sqrt(D)).
template <int D, bool kDiag>
__device__ __forceinline__ float tile_scores(const u32x4_t (&kr)[D / 8], const uint4 (&qreg)[D / 16],
                                             f32x16_t (&sacc)[2], int q_local, int hl, float c) {
  sacc[0] = f32x16_t{};
  sacc[1] = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      sacc[mt] = mfma_32x32x16(__builtin_bit_cast(uint4, kr[2 * ks + mt]), qreg[ks], sacc[mt]);
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
  return pair_max(mx) * c;
}

// Online-softmax update with one tile: lazy rescale (the running max m moves
// only when a lane's tile max exceeds it by more than the slack), P = exp2(s c
// - m) packed to bf16 in the B-operand layout, and O^T += V^T P^T.
// As tile_scores with the diagonal decided at run time (one inlined copy in a
// loop). The causality compares take the query row through an empty asm so
// that they are not hoisted out of the loop as 32 loop-invariant scalar masks.
template <int D>
__device__ __forceinline__ float tile_scores_rt(const u32x4_t (&kr)[D / 8], const uint4 (&qreg)[D / 16],
                                                f32x16_t (&sacc)[2], int q_local, int hl, float c, bool diag) {
  sacc[0] = f32x16_t{};
  sacc[1] = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      sacc[mt] = mfma_32x32x16(__builtin_bit_cast(uint4, kr[2 * ks + mt]), qreg[ks], sacc[mt]);
  if (diag) {
    int ql = q_local - 4 * hl;
    asm volatile("" : "+v"(ql));
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * mt + 8 * (r >> 2) + (r & 3);
        if (key > ql) sacc[mt][r] = -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mt][r]);
  return pair_max(mx) * c;
}

template <int D>
__device__ __forceinline__ void tile_update(const f32x16_t (&sacc)[2], const u32x2_t (&vr)[D / 4], float mx,
                                            float c, float& m, float& lsum, f32x16_t (&oacc)[D / 32]) {
  constexpr int MT = D / 32;
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
}

// The block-sparse kernels split tile_scores / tile_update by the tile's place
// in the row. The row's first tile (m = -inf on entry, the diagonal when it
// is active) takes its maximum, which becomes m, and skips the rescale of the
// still-zero accumulators. A later tile skips its maximum unless it could move
// m: P = exp2(s c - m) is computed under the current m first, and only when
// some lane's probabilities sum past kLazyCheck is the maximum taken and the
// rescale rule of tile_update applied (and P recomputed if m moved). A score
// that exceeds m by the slack (8) has P > 2^7.9 > kLazyCheck, so every tile
// that tile_update would rescale takes that branch, and every other tile
// keeps the P it computed under the unchanged m: the results are bitwise those
// of tile_scores + tile_update, with 16 v_max3, the pair max, the scaling and
// the compare gone from most tiles.
constexpr float kLazyCheck = 64.0f;

// S^T = K Q^T for one tile without its row maximum.
template <int D>
__device__ __forceinline__ void tile_qk(const u32x4_t (&kr)[D / 8], const uint4 (&qreg)[D / 16],
                                        f32x16_t (&sacc)[2]) {
  sacc[0] = f32x16_t{};
  sacc[1] = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      sacc[mt] = mfma_32x32x16(__builtin_bit_cast(uint4, kr[2 * ks + mt]), qreg[ks], sacc[mt]);
}

// P = exp2(s c - m) packed to bf16 in the B-operand layout of O^T = V^T P^T
// (the order of tile_update), and the lane's sum of P
__device__ __forceinline__ float tile_probs(const f32x16_t (&sacc)[2], float c, float m, uint4 (&pb)[4]) {
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
  return ls;
}

template <int D>
__device__ __forceinline__ void tile_pv(const u32x2_t (&vr)[D / 4], const uint4 (&pb)[4], f32x16_t (&oacc)[D / 32]) {
  constexpr int MT = D / 32;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x2_t lo = vr[(ks * MT + mt) * 2], hi = vr[(ks * MT + mt) * 2 + 1];
      oacc[mt] = mfma_32x32x16(make_uint4(lo.x, lo.y, hi.x, hi.y), pb[ks], oacc[mt]);
    }
}

// First tile of a row: m = -inf, lsum = 0 and oacc = 0 on entry; mx is the
// tile's maximum from tile_scores (finite: the row's first tile holds a
// causal key for every query). Leaves P in pb.
__device__ __forceinline__ void tile_softmax_first(const f32x16_t (&sacc)[2], float mx, float c, float& m,
                                                   float& lsum, uint4 (&pb)[4]) {
  m = mx;
  lsum = tile_probs(sacc, c, m, pb);
}

// A later tile of a row (see kLazyCheck). Leaves P in pb.
template <int D>
__device__ __forceinline__ void tile_softmax_lazy(const f32x16_t (&sacc)[2], float c, float& m, float& lsum,
                                                  f32x16_t (&oacc)[D / 32], uint4 (&pb)[4]) {
  constexpr int MT = D / 32;
  float ls = tile_probs(sacc, c, m, pb);
  if (__builtin_amdgcn_ballot_w64(ls > kLazyCheck)) {
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mt][r]);
    mx = pair_max(mx) * c;
    const bool upd = mx > m + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(upd)) {
      const float mn = upd ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < MT; ++i) oacc[i] *= alpha;
      m = mn;
      ls = tile_probs(sacc, c, m, pb);
    }
  }
  lsum += ls;
}

// A row's output over its key chunks: O = sum_c w_c O_c / sum_c w_c, w_c =
// 2^(L_c - max L), over the chunk in registers (oacc unnormalized, its inv and
// log2-sum-exp lse2 on entry) and the row's partials of chunks [0, chunk),
// normalized bf16 outputs and log2-sum-exps that attn_sparse_xcd_kernel wrote
// to the workspace: the 8-value group g of thread tid (oacc[g / 2] values
// 8 (g % 2) ..) is 16 bytes at uint4 index g * kThreads + tid of the slot,
// the register layout here. On return oacc holds the weighted sum, inv and
// lse2 the row's. One pass with a running maximum: the slots are loaded
// kSlots at a time with their log2-sum-exps, all loads of a batch issued
// before any is used, and the sum so far is rescaled when a batch raises the
// maximum, so a row waits for one memory round trip per batch.
template <int D, int kSlots>
__device__ __forceinline__ void merge_chunk_partials(const AttnArgs& p, int bh, int qb, int chunk, int tid,
                                                     int q_local, f32x16_t (&oacc)[D / 32], float& inv,
                                                     float& lse2) {
  constexpr int MT = D / 32;
  constexpr int NG = 2 * MT;                  // 16-byte groups per thread and slot
  const long long slot0 = static_cast<long long>(bh) * p.slots_per_head + xcd_slot_base(qb, p.chunk);
  const float* lsl = p.part_l + slot0 * kBlock + q_local;
  const uint4* src = reinterpret_cast<const uint4*>(p.part_o16 + slot0 * kBlock * D) + tid;
  // running state: maximum M, wsum = sum_c 2^(L_c - M), oacc = sum_c 2^(L_c - M) O_c
  float mrun = lse2, wsum;
  if (lse2 > -INFINITY) {
    wsum = 1.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oacc[mt] *= inv;
  } else {
    wsum = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oacc[mt] = f32x16_t{};
  }
  for (int c0 = 0; c0 < chunk; c0 += kSlots) {
    uint4 v[kSlots][NG];
    float wl[kSlots];
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      const bool ok = c0 + u < chunk;
      const int cc = ok ? c0 + u : c0;          // a slot that exists; its weight is 0 below
      wl[u] = ok ? lsl[cc * kBlock] : -INFINITY;
#pragma unroll
      for (int g = 0; g < NG; ++g) v[u][g] = src[static_cast<long long>(cc) * (kBlock * D / 8) + g * kThreads];
    }
    float mnew = mrun;
#pragma unroll
    for (int u = 0; u < kSlots; ++u) mnew = fmaxf(mnew, wl[u]);
    if (mnew == -INFINITY) continue;            // nothing so far has a key
    if (mnew > mrun) {                          // the batch raises the maximum: rescale the sum so far
      const float sc = __builtin_amdgcn_exp2f(mrun - mnew);   // 0 while mrun = -inf
      wsum *= sc;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) oacc[mt] *= sc;
      mrun = mnew;
    }
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      const float wu = __builtin_amdgcn_exp2f(wl[u] - mrun);
      wsum += wu;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const uint32_t wd[4] = {v[u][g].x, v[u][g].y, v[u][g].z, v[u][g].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i0 = 8 * (g % 2) + 2 * e;
          oacc[g / 2][i0] = fmaf(wu, __uint_as_float(wd[e] << 16), oacc[g / 2][i0]);
          oacc[g / 2][i0 + 1] = fmaf(wu, __uint_as_float(wd[e] & 0xffff0000u), oacc[g / 2][i0 + 1]);
        }
      }
    }
  }
  inv = wsum > 0.f ? 1.f / wsum : 0.f;
  lse2 = wsum > 0.f ? mrun + __log2f(wsum) : -INFINITY;
}

// Called twice per row: hook(0) during the row's last tile, once its V copy is
// issued (at the end of a row without tiles), and hook(1) before the row's
// output stores. attn_sparse_rows_kernel claims its next row at the first
// and hands the claim to its workgroup at the second. The other kernels pass
// nothing.
struct NoRowHook {
  __device__ void operator()(int) const {}
};

// One (batch, query head, query block) row -- or one key chunk of it -- of
// the tile loop below. `w` is the row's workgroup index in the launch (its
// claim index in a persistent launch) the block-sparse circular sweep is
// phased by (see the sweep below).
template <int D, int MODE, typename Hook = NoRowHook>
__device__ __forceinline__ void attn_row(const AttnArgs& p, const int w, const int qb, const int bh,
                                         const int chunk, Hook hook = Hook{}) {
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

  // the diagonal tile is processed first; start its K copy before anything
  // else (in block-sparse mode only the item whose chunk holds the diagonal
  // has it)
  if (MODE != kSparse || qb < (chunk + 1) * p.chunk) issue_k(qb);

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

  // One tile kb. On entry its K copy is in flight or landed and its V copy is
  // not issued yet. Two workgroup barriers per tile: the one that publishes
  // K(kb) also frees the V buffer (both waves have read the previous tile's
  // V), so V(kb) is copied from there on; the one that publishes V(kb) frees
  // the K buffer, so K(next) is copied from there on. Each batch of copies is
  // issued while the wave's operand reads from LDS are in flight. Both waits
  // are for everything outstanding: the ground-truth row-max store of a tile
  // is issued after the second one, so the next tile's first wait covers it.
  // kFirst: the row's first tile (the diagonal when it is active), which sets
  // the running max; later tiles take their maximum only when it could move
  // it (tile_softmax_lazy), except in ground-truth mode, which records every
  // tile's maximum.
  auto compute = [&](auto diag_tag, auto first_tag, int kb, int next) {
    constexpr bool kDiag = decltype(diag_tag)::value;   // the diagonal tile needs element causality
    constexpr bool kFirst = decltype(first_tag)::value;
    constexpr bool kLazy = MODE != kDenseGt && !kFirst;
    wait_vm(0);                                    // K(kb) landed, and every copy and store before it
    wg_barrier();
    u32x4_t kr[2 * KS];                           // kr[2 ks + mt]: keys 32 mt + l32, dims 16 ks + 8 hl ..
    read_k_issue<D>(kaddr, kr);
    issue_v(kb);
    if (next < 0) hook(0);                         // the row's last tile
    read_k_wait<D>(kr);

    f32x16_t sacc[2];
    float mx = 0.f;
    uint4 pb[4];
    if constexpr (kLazy) {
      static_assert(!kDiag, "the diagonal tile is a row's first");
      tile_qk<D>(kr, qreg, sacc);
      tile_softmax_lazy<D>(sacc, c, m, lsum, oacc, pb);
    } else {
      mx = tile_scores<D, kDiag>(kr, qreg, sacc, q_local, hl, c);
      if constexpr (kFirst) tile_softmax_first(sacc, mx, c, m, lsum, pb);
    }

    wait_vm(0);                                    // V(kb) landed
    wg_barrier();
    if constexpr (MODE == kDenseGt) {
      if (hl == 0) p.rmax[((static_cast<size_t>(bh) * p.ntri + ntri_off + kb) << 6) + q_local] = mx;
    }
    u32x2_t vr[8 * MT];                            // vr[(ks MT + mt) 2 + u]: dims 32 mt + .., keys 16 ks + 8 u + ..
    read_v_issue<D>(vaddr, vr);
    if (next >= 0) issue_k(next);
    read_v_wait<D>(vr);

    if constexpr (kLazy || kFirst) tile_pv<D>(vr, pb, oacc);
    else tile_update<D>(sacc, vr, mx, c, m, lsum, oacc);
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
    // to this workgroup's place in its XCD's dispatch sequence (kSweepPhases
    // phases) and wraps around. Workgroups of one XCD start one after
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
      compute(std::true_type{}, std::true_type{}, qb, nxt);
      issued = cnt > 0;
    } else if (has_diag) {
      wait_vm(0);                            // the early copy of the diagonal tile is not used
      wg_barrier();
    }
    if (cnt > 0) {
      int kb = entry(0);
      if (!issued) issue_k(kb);
      int n = 0;
      if (!diag_on) {                          // the sweep's first tile is the row's first
        const int next = cnt > 1 ? entry(1) : -1;
        compute(std::false_type{}, std::true_type{}, kb, next);
        kb = next;
        n = 1;
      }
      for (; n < cnt; ++n) {
        const int next = n + 1 < cnt ? entry(n + 1) : -1;
        compute(std::false_type{}, std::false_type{}, kb, next);
        kb = next;
      }
    }
    if (cnt == 0 && !diag_on) hook(0);
  } else {
    compute(std::true_type{}, std::true_type{}, qb, qb > 0 ? 0 : -1);
    for (int kb = 0; kb < qb; ++kb) compute(std::false_type{}, std::false_type{}, kb, kb + 1 < qb ? kb + 1 : -1);
  }

  // ---- epilogue: normalize, store O and LSE --------------------------------
  hook(1);
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

// Pre-pass of the XCD-major row order: active causal tiles of the mask rows
// [16 y, 16 y + 16) of flattened head bh = blockIdx.x, added to the count of
// the XCD that owns the head in that order (xcd_work, zeroed before).
constexpr int kWorkRows = 16;
__global__ __launch_bounds__(256) void attn_xcd_work_kernel(AttnArgs p) {
  const int bh = blockIdx.x;
  const int q0 = blockIdx.y * kWorkRows;
  const int rows = min(kWorkRows, p.nb - q0);
  const uint8_t* m = p.mask + (static_cast<size_t>(bh) * p.nb + q0) * p.nb;
  const int n = rows * p.nb;
  int cnt = 0;
#pragma unroll 8
  for (int e = threadIdx.x; e < n; e += 256) {
    const int r = e / p.nb;
    cnt += (e - r * p.nb <= q0 + r && m[e] != 0) ? 1 : 0;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
  __shared__ int part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicAdd(p.xcd_work + bh / (p.B * p.Hq / kXcds), part[0] + part[1] + part[2] + part[3]);
}

// Block-sparse rows of one item in a persistent launch: kRowSlots
// workgroups per XCD (its resident capacity). Queue y holds the rows of the
// flattened heads [h0(y), h0(y+1)), h0(y) = y B Hq / 8, query block descending
// with the heads interleaved, and the workgroups of XCD x take their rows from
// queue x in order, so each XCD's L2 serves its own heads' KV groups. Slot s
// starts with row s of its queue (the counters start at kRowSlots); each later
// row is claimed from a per-queue counter during the current row's last tile.
// A workgroup whose queue has run dry takes its rows from the queue with the
// most rows left (the heads' masks can give one XCD half again the mean work),
// and ends once every queue is dry.
constexpr int kRowSlots = 128;             // resident workgroups per XCD: 32 CUs x 4
__device__ __forceinline__ int rows_h0(const AttnArgs& p, int y) { return (y * p.B * p.Hq) / kXcds; }
__device__ __forceinline__ int rows_queue_len(const AttnArgs& p, int y) {
  return (rows_h0(p, y + 1) - rows_h0(p, y)) * p.nb;
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_sparse_rows_kernel(AttnArgs p) {
  constexpr int kNone = 0x7fffffff;
  __shared__ int claim_s[2];
  const int tid = threadIdx.x;
  const int x = static_cast<int>(blockIdx.x % kXcds);
  int y = x;                                       // the queue this workgroup claims from
  int n = rows_queue_len(p, y);
  int j = static_cast<int>(blockIdx.x / kXcds);    // its first row: row s of queue x
  while (true) {
    if (j >= n) {
      // queue y is dry: wave 0 reads every queue's counter (device-scope
      // loads: the counters move on other XCDs) and claims from the queue
      // with the most rows left, or the workgroup ends
      if (tid < kWave) {
        int rem = -1;
        if (tid < kXcds)
          rem = rows_queue_len(p, tid) - __hip_atomic_load(p.xcd_ctr + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int best = rem, by = tid;
#pragma unroll
        for (int o = 1; o < kXcds; o <<= 1) {
          const int ob = __shfl_xor(best, o), oy = __shfl_xor(by, o);
          if (ob > best || (ob == best && oy < by)) {
            best = ob;
            by = oy;
          }
        }
        if (tid == 0) {
          claim_s[0] = by;
          claim_s[1] = best > 0 ? atomicAdd(p.xcd_ctr + by, 1) : kNone;
        }
      }
      __syncthreads();
      y = __builtin_amdgcn_readfirstlane(claim_s[0]);
      j = __builtin_amdgcn_readfirstlane(claim_s[1]);
      __syncthreads();                             // both waves hold them before the LDS words are reused
      if (j == kNone) return;
      n = rows_queue_len(p, y);
      continue;
    }
    const int h0 = rows_h0(p, y);
    const int nh = rows_h0(p, y + 1) - h0;
    const int i = j / nh;
    int pend = 0;                                  // thread 0: the claim in flight
    int* const cy = p.xcd_ctr + y;
    auto hook = [&](int stage) {
      if (tid != 0) return;
      if (stage == 0) {
        // an address the compiler cannot prove uniform: a uniform one makes
        // it read the result back at once
        int off = 0;
        asm volatile("" : "+v"(off));
        pend = atomicAdd(cy + off, 1);
      } else {
        claim_s[1] = pend;
      }
    };
    // the sweep's phase is the claim index modulo kSweepPhases
    attn_row<D, kSparse>(p, (j % kSweepPhases) * kXcds, p.nb - 1 - i, h0 + (j - i * nh), 0, hook);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    wg_barrier();
    j = __builtin_amdgcn_readfirstlane(static_cast<int>(lds_read_u32(lds_addr(&claim_s[1]))));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    wg_barrier();                                  // both waves hold it before the LDS word is reused
  }
}

// Counters of attn_sparse_rows_kernel: each queue's first kRowSlots rows are
// the slots' first rows.
__global__ void attn_rows_counters_init(int* ctr) {
  if (threadIdx.x < kXcds) ctr[threadIdx.x] = kRowSlots;
}

template <int D, int MODE>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(AttnArgs p) {
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
  bool xcd_major = false;
  if constexpr (MODE == kSparse) {
    if (p.xcd_work != nullptr) {
      // balanced when the most loaded XCD has at most 1.2 x the mean
      long long mx = 0, sum = 0;
#pragma unroll
      for (int x = 0; x < kXcds; ++x) {
        const long long cx = static_cast<unsigned>(p.xcd_work[x]);
        mx = max(mx, cx);
        sum += cx;
      }
      xcd_major = 5 * kXcds * mx <= 6 * sum;
    }
  }
  if (MODE == kSparse && xcd_major) {
    // Rows of one item, query block descending (the longest rows first);
    // within a query block, the workgroups that land on XCD x take the heads
    // [x BH/8, (x+1) BH/8), so each XCD's L2 serves the K/V of those heads'
    // groups only. Each XCD then does the work of its heads, so this order
    // is taken only when the pre-pass found those counts balanced; the host
    // asks for it only for short rows and B Hq a multiple of 8.
    const int per = BH / kXcds;
    qb = p.nb - 1 - w / BH;
    const int local = w % BH;
    bh = (local % kXcds) * per + local / kXcds;
  } else if constexpr (MODE == kSparse) {
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
  attn_row<D, MODE>(p, w, qb, bh, chunk);
}

// ---------------------------------------------------------------------------
// Dense causal attention (and its ground-truth variant) for GQA groups of a
// multiple of four query heads: one workgroup = four query heads of one KV
// group at one query block, 8 wavefronts (head-major, two 32-query halves
// per head). The four heads read the same K/V tiles, so each tile is copied
// HBM -> LDS once for 256 queries instead of once per 64, and the LDS that
// four row-workgroups would use holds a ring of kRing tiles: the copies run
// kRing - 1 tiles ahead, and one workgroup barrier per tile both publishes
// the tile every wave copied a part of and frees the slot of the tile before.
// Each wavefront does exactly what a wavefront of attn_fwd_kernel does for
// its 32 queries (same tile order, same tile arithmetic), so results are
// bitwise those of attn_fwd_kernel.
constexpr int kGqaHeads = 4;                 // query heads per workgroup
constexpr int kGqaWaves = 2 * kGqaHeads;
constexpr int kGqaThreads = kGqaWaves * kWave;
constexpr int kRing = 4;                     // K/V tiles in flight per workgroup

template <int D, int MODE>
__device__ __forceinline__ void attn_dense_gqa_body(const AttnArgs& p) {
  static_assert(MODE != kSparse, "dense modes only");
  constexpr int CPR = D / 8;                 // 16-byte chunks per K/V row
  constexpr int KS = D / 16;
  constexpr int MT = D / 32;
  constexpr int RPI = 64 / CPR;              // tile rows per copy instruction
  constexpr int NCW = (kBlock / kGqaWaves) / RPI;   // copy instructions per wave per operand and tile
  constexpr int TILE_BYTES = kBlock * CPR * 16;     // one K or V tile
  static_assert(NCW >= 1 && (kBlock / kGqaWaves) % RPI == 0, "copy split");

  __shared__ uint4 Kr[kRing * kBlock * CPR];
  __shared__ uint4 Vr[kRing * kBlock * CPR];
  __shared__ float lse_s[MODE == kDenseGt ? kGqaHeads * kBlock : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int hloc = wave >> 1;                // head within the workgroup
  const int q_local = (wave & 1) * 32 + l32; // query row within the block

  // workgroups: (batch, KV group, 4-head quarter) major, query block descending
  const int quarters = p.group / kGqaHeads;
  const int per_q = p.nb;
  const int w = blockIdx.x;
  const int gq = w / per_q;                  // (b * Hkv + g) * quarters + quarter
  const int qb = p.nb - 1 - (w - gq * per_q);
  const int bg = gq / quarters;
  const int b = bg / p.Hkv;
  const int g = bg - b * p.Hkv;
  const int h = g * p.group + (gq - bg * quarters) * kGqaHeads + hloc;
  const int bh = b * p.Hq + h;
  const size_t kv_off = (static_cast<size_t>(b) * p.Hkv + g) * p.hs * D;
  const uint16_t* __restrict__ Kg = p.k + kv_off;
  const uint16_t* __restrict__ Vg = p.v + kv_off;

  // this wave copies rows 8 wave .. 8 wave + 7 of every tile: instruction i,
  // lane l moves tile row r = 8 wave + RPI i + l / CPR, physical chunk l % CPR
  // holding logical chunk (l % CPR) ^ swz(r), to LDS byte 1024 (NCW wave + i) + 16 l
  uint32_t kofs[NCW], vofs[NCW];
#pragma unroll
  for (int i = 0; i < NCW; ++i) {
    const int r = 8 * wave + RPI * i + lane / CPR;
    const int pc = lane % CPR;
    kofs[i] = static_cast<uint32_t>(r * 2 * D + 16 * (pc ^ swz_k<D>(r)));
    vofs[i] = static_cast<uint32_t>(r * 2 * D + 16 * (pc ^ swz_v<D>(r)));
  }
  auto issue = [&](int kb, int slot) {
    const int key0 = kb * kBlock;
    const uint32_t bytes = static_cast<uint32_t>((p.S - key0) * 2 * D);
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Kg + static_cast<size_t>(key0) * D), 0,
                                                      bytes, kBufferWord3);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Vg + static_cast<size_t>(key0) * D), 0,
                                                      bytes, kBufferWord3);
    char* kd = reinterpret_cast<char*>(Kr) + slot * TILE_BYTES + 1024 * NCW * wave;
    char* vd = reinterpret_cast<char*>(Vr) + slot * TILE_BYTES + 1024 * NCW * wave;
#pragma unroll
    for (int i = 0; i < NCW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(kd + 1024 * i), 16, kofs[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < NCW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(vd + 1024 * i), 16, vofs[i], 0, 0, 0);
  };

  // operand read addresses in slot 0 (the swizzles of attn_fwd_kernel)
  uint32_t kaddr0[KS], vaddr0[MT];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    kaddr0[ks] = lds_addr(Kr) + l32 * 2 * D + 16 * ((2 * ks + hl) ^ swz_k<D>(l32));
  {
    const int G = lane >> 4, jj = (lane >> 2) & 3, a = lane & 3;
    const int key = 4 * (G >> 1) + jj;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      vaddr0[mt] = lds_addr(Vr) + key * 2 * D + 16 * ((4 * mt + 2 * (G & 1) + (a >> 1)) ^ swz_v<D>(key)) + 8 * (a & 1);
  }

  // tiles in the order of attn_fwd_kernel: the diagonal first, then 0 .. qb - 1
  const int ntiles = qb + 1;
  auto tile_kb = [&](int t) { return t == 0 ? qb : t - 1; };
  // Vector-memory operations of this wave, in issue order: the copies of
  // tiles 0 .. pro-1 (kPerTile each), the KS Q loads, then per tile t: the
  // copies of tile t + kRing - 1 (while that tile exists) and, for the ground
  // truth, one store. Before tile t is read the wave waits until at most
  // issued(t) - after(t) operations are outstanding: issued(t) counts all it
  // issued before tile t, after(t) those up to and including tile t's copies.
  constexpr int kPerTile = 2 * NCW;          // copy instructions per wave and tile
  constexpr int kStore = MODE == kDenseGt ? 1 : 0;
  const int pro = ntiles < kRing - 1 ? ntiles : kRing - 1;
  const int late = ntiles - (kRing - 1) > 0 ? ntiles - (kRing - 1) : 0;   // tiles copied inside the loop
  auto issued_before = [&](int t) { return (pro + (t < late ? t : late)) * kPerTile + KS + t * kStore; };
  auto through_copies = [&](int t) {
    if (t < pro) return (t + 1) * kPerTile;
    const int i = t - (kRing - 1);           // the tile whose step issued these copies
    return (pro + i + 1) * kPerTile + KS + i * kStore;
  };
  for (int t = 0; t < pro; ++t) issue(tile_kb(t), t);

  // Q fragment of this wave's 32 queries
  const int t_q = qb * kBlock + q_local;
  const bool t_ok = t_q < p.S;
  uint4 qreg[KS];
  {
    const uint16_t* qrow = p.q + (static_cast<size_t>(bh) * p.hs + (t_ok ? t_q : 0)) * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[ks] = t_ok ? *reinterpret_cast<const uint4*>(qrow + 16 * ks) : make_uint4(0, 0, 0, 0);
  }

  const float c = p.scale_log2;
  float m = -INFINITY, lsum = 0.f;
  f32x16_t oacc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) oacc[i] = f32x16_t{};
  const long long ntri_off = static_cast<long long>(qb) * (qb + 1) / 2;

  auto step = [&](auto diag_tag, int t) {
    constexpr bool kDiag = decltype(diag_tag)::value;
    const int slot = t % kRing;
    const int kb = tile_kb(t);
    wait_vm_upto(issued_before(t) - through_copies(t));   // this wave's part of tile t landed
    wg_barrier();                            // every part landed; every wave is done with tile t - 1

    const uint32_t off = static_cast<uint32_t>(slot * TILE_BYTES);
    uint32_t kaddr[KS], vaddr[MT];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kaddr[ks] = kaddr0[ks] + off;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) vaddr[mt] = vaddr0[mt] + off;
    u32x4_t kr[2 * KS];
    read_k_issue<D>(kaddr, kr);
    if (t + kRing - 1 < ntiles) {            // refill the slot of tile t - 1 while the K reads are in flight
      const int tn = t + kRing - 1;
      issue(tile_kb(tn), tn % kRing);
    }
    read_k_wait<D>(kr);
    f32x16_t sacc[2];
    const float mx = tile_scores<D, kDiag>(kr, qreg, sacc, q_local, hl, c);
    if constexpr (MODE == kDenseGt) {
      if (hl == 0) p.rmax[((static_cast<size_t>(bh) * p.ntri + ntri_off + kb) << 6) + q_local] = mx;
    }
    u32x2_t vr[8 * MT];
    read_v_tile<D>(vaddr, vr);
    tile_update<D>(sacc, vr, mx, c, m, lsum, oacc);
  };
  step(std::true_type{}, 0);
  for (int t = 1; t < ntiles; ++t) step(std::false_type{}, t);

  // ---- epilogue: normalize, store O and LSE (as attn_fwd_kernel)
  const float ltot = pair_sum(lsum);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  const float lse2 = ltot > 0.f ? m + __log2f(ltot) : -INFINITY;
  if (t_ok) {
    const size_t obase = (static_cast<size_t>(bh) * p.hs + t_q) * D;
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
    if (p.lse != nullptr && hl == 0) p.lse[static_cast<size_t>(bh) * p.hs + t_q] = lse2 * kLn2;
  }

  if constexpr (MODE == kDenseGt) {
    // gt[qb, kb] = max over the block's queries of exp2(r - lse2) per head; 0 above the diagonal
    if (hl == 0) lse_s[hloc * kBlock + q_local] = t_ok ? lse2 : INFINITY;
    __syncthreads();                         // lse_s and the heads' r writes visible to the workgroup
    const int bh0 = bh - hloc;               // first head of the workgroup
    for (int e = tid; e < kGqaHeads * p.nb; e += kGqaThreads) {
      const int hh = e / p.nb, kb = e - hh * p.nb;
      float best = 0.f;
      if (kb <= qb) {
        const float4* rr = reinterpret_cast<const float4*>(
            p.rmax + ((static_cast<size_t>(bh0 + hh) * p.ntri + ntri_off + kb) << 6));
        const float* ls = lse_s + hh * kBlock;
#pragma unroll 4
        for (int q4 = 0; q4 < 16; ++q4) {
          const float4 v = rr[q4];
          best = fmaxf(best, exp2f(v.x - ls[4 * q4 + 0]));
          best = fmaxf(best, exp2f(v.y - ls[4 * q4 + 1]));
          best = fmaxf(best, exp2f(v.z - ls[4 * q4 + 2]));
          best = fmaxf(best, exp2f(v.w - ls[4 * q4 + 3]));
        }
      }
      p.gt[(static_cast<size_t>(bh0 + hh) * p.nb + qb) * p.nb + kb] = best;
    }
  }
}

template <int D, int MODE>
__global__ __launch_bounds__(kGqaThreads, 1) void attn_dense_gqa_kernel(AttnArgs p) {
  attn_dense_gqa_body<D, MODE>(p);
}

// Packed (varlen) batch in one launch: workgroup w takes a row of the sequence
// whose row range holds w. Each sequence is the batch-1 problem at its token
// offset with the packed length as head stride, and every row runs exactly
// what the batch-1 call on that sequence runs for it (the block-sparse sweep
// is phased by the row's workgroup index in that call), so the results are
// bitwise those of the batch-1 calls. Rows of a sequence go in the batch-1
// order; sequences in table order (longest first).
template <int D, int MODE>
__global__ __launch_bounds__(kThreads, 2) void attn_varlen_kernel(AttnArgs p, VarlenTable t) {
  const int w = blockIdx.x;
  int lo = 0, hi = t.n - 1;                       // last sequence i with row_start[i] <= w
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (t.row_start[mid] <= w) lo = mid;
    else hi = mid - 1;
  }
  AttnArgs a = p;
  const size_t tok = static_cast<size_t>(t.tok[lo]);
  a.q += tok * D;
  a.k += tok * D;
  a.v += tok * D;
  a.out = a.out_bf16 ? static_cast<void*>(static_cast<uint16_t*>(p.out) + tok * D)
                     : static_cast<void*>(static_cast<float*>(p.out) + tok * D);
  if (a.lse != nullptr) a.lse += tok;
  a.S = t.len[lo];
  a.nb = (a.S + kBlock - 1) / kBlock;
  a.ntri = static_cast<long long>(a.nb) * (a.nb + 1) / 2;
  if constexpr (MODE == kSparse) {
    a.mask += t.map_off[lo];
    a.items_per_group = static_cast<long long>(a.group) * a.nb;
  }
  if constexpr (MODE == kDenseGt) {
    a.gt += t.map_off[lo];
    a.rmax += t.rmax_off[lo];
  }
  // the row's place in the batch-1 launch order: KV-group major (one group's
  // K/V hot at a time), then head-major for block-sparse rows, query-block
  // major for dense ones, heaviest rows first
  const int local = w - t.row_start[lo];
  const int per_group = a.group * a.nb;
  const int g = local / per_group, r = local - g * per_group;
  int qb, hig;
  if constexpr (MODE == kSparse) {
    hig = r / a.nb;
    qb = a.nb - 1 - (r - hig * a.nb);
  } else {
    qb = a.nb - 1 - r / a.group;
    hig = r - (a.nb - 1 - qb) * a.group;
  }
  attn_row<D, MODE>(a, local, qb, g * a.group + hig, 0);
}

// ---------------------------------------------------------------------------
// Block-sparse rows of many key blocks: XCD-owned key chunks, persistent
// workgroups.
//
// The key range is cut into chunks of C blocks. A job is one chunk of one
// (batch, KV group): the (row, chunk) items of every query head of the group
// whose rows lie past the chunk, head major, query block descending. The
// chunk that holds a row's diagonal is an item of a second launch of the same
// kernel (kDiagPhase, after the first has finished, with the same jobs holding
// the rows inside their chunk instead): it writes the row's output, merging
// its own chunk (in registers) with the row's partials of the earlier chunks
// in its epilogue, where the merge's loads from HBM run under the tiles of the
// other workgroups on the CU.
// Jobs are dealt to the 8 XCDs in the order 0..7, 7..0, 0..7, ... (so each XCD
// gets chunks c and n-1-c of the groups, which evens out the causal triangle)
// and every XCD works through its own jobs one after another: the K/V of the
// chunk its items read (C = 128 tiles of 32 KiB at D = 128, the size of the
// XCD's 4 MiB L2) is fetched from HBM a few times per job instead of once per
// reading row. The
// grid is the resident capacity, kXcdSlots workgroups per XCD; workgroup w
// runs on XCD w % 8 and takes the next item of that XCD's sequence from a
// per-XCD counter, so the items resident on an XCD stay a contiguous window of
// its sequence (a fixed stride per workgroup lets them drift over several
// chunks). Nothing drains between items: item indices are fetched two items
// ahead, the next item's mask flags one item ahead, and its Q rows and the K
// of its first tile are issued during the current item's last tile. Every
// item of the first launch writes a bf16 partial output (normalized by its own
// sum) and its log2-sum-exp.
constexpr int kXcdDefaultChunk = 128;    // 4 MiB of K/V at D = 128: one XCD's L2
static_assert(kXcdDefaultChunk <= 128, "an item's flags are two 64-bit ballot words");
constexpr int kXcdMinBlocks = 960;       // rows of 60k tokens and more
constexpr int kXcdSlots = 128;           // resident workgroups per XCD: 32 CUs x 4


// Job at position t of XCD x's sequence, or -1 past its end. Positions 2i and
// 2i+1 take jobs 16i + x and 16i + 15 - x; the first job past the end ends it.
__device__ __forceinline__ int xcd_job(int x, int t, int njobs) {
  const int base = 2 * kXcds * (t >> 1);
  const int k = (t & 1) ? base + 2 * kXcds - 1 - x : base + x;
  return k < njobs ? k : -1;
}

struct XcdItem {
  int bh;          // batch * Hq + head; -1: past the end of the sequence
  int qb;          // query block
  int c;           // key chunk
  long long kvo;   // element offset of the item's K/V head
};

// Walks one XCD's item sequence; queried with non-decreasing item indices
// (the host keeps every index within 32 bits). What depends only on the job
// is computed once, when the walk enters the job; within a job the head
// advances incrementally, so an item costs no integer division (the scalar
// arithmetic of an item start issues at one instruction per four cycles).
struct XcdCursor {
  int t = 0;               // position in the XCD's job sequence
  int job = -1;
  int begin = 0;           // sequence index of the job's first item
  int count = 0;           // items in the job
  int c = 0;               // the job's key chunk
  int rows = 0;            // query blocks per head that reach the chunk
  int bh0 = 0;             // batch * Hq + first query head of the job's KV group
  int hig = 0;             // head within the group of the last item returned
  int hbase = 0;           // job-relative index of that head's first item
  long long kvo = 0;       // element offset of the job's K/V head
};

template <int D, bool kDiagPhase>
__device__ __forceinline__ XcdItem xcd_item(const AttnArgs& p, int x, int j, XcdCursor& cur) {
  while (true) {
    if (cur.job < 0) {
      cur.job = xcd_job(x, cur.t, p.njobs);
      if (cur.job < 0) return XcdItem{-1, 0, 0, 0};
      cur.c = cur.job % p.nchunk;
      const int gi = cur.job / p.nchunk;
      const int bb = gi / p.Hkv, gg = gi - bb * p.Hkv;
      // rows past the chunk; in the diagonal phase the rows inside it
      cur.rows = kDiagPhase ? min(p.nb - cur.c * kXcdDefaultChunk, kXcdDefaultChunk)
                            : max(p.nb - (cur.c + 1) * kXcdDefaultChunk, 0);
      cur.count = p.group * cur.rows;
      cur.bh0 = bb * p.Hq + gg * p.group;
      cur.kvo = (static_cast<long long>(bb) * p.Hkv + gg) * p.hs * D;
      cur.hig = 0;
      cur.hbase = 0;
    }
    if (j < cur.begin + cur.count) break;
    cur.begin += cur.count;
    ++cur.t;
    cur.job = -1;
  }
  const int mi = j - cur.begin;
  if constexpr (kDiagPhase) {
    // query block major, ascending, the group's heads in turn: the items
    // resident on the XCD read the K/V of the chunk's first blocks up to
    // about their own query block, and the heads of one query block read the
    // same tiles at the same time
    const int r = mi / p.group;
    return XcdItem{cur.bh0 + (mi - r * p.group), cur.c * kXcdDefaultChunk + r, cur.c, cur.kvo};
  } else {
    while (mi >= cur.hbase + cur.rows) {
      cur.hbase += cur.rows;
      ++cur.hig;
    }
    return XcdItem{cur.bh0 + cur.hig, p.nb - 1 - (mi - cur.hbase), cur.c, cur.kvo};   // query blocks descending
  }
}


template <int D, bool kDiagPhase>
__global__ __launch_bounds__(kThreads, 2) void attn_sparse_xcd_kernel(AttnArgs p) {
  constexpr int CPR = D / 8;               // 16-byte chunks per K/V row
  constexpr int KS = D / 16;               // MFMA k-steps for S^T (= Q loads per thread)
  constexpr int MT = D / 32;               // MFMA m-tiles for O^T
  constexpr int RPI = 64 / CPR;            // tile rows per copy instruction
  constexpr int NDMA = 32 / RPI;           // copy instructions per wave per operand

  __shared__ uint4 Ks[kBlock * CPR];
  __shared__ uint4 Vs[kBlock * CPR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int q_local = wave * 32 + l32;
  const int x = static_cast<int>(blockIdx.x % kXcds);
  int* const ctr = p.xcd_ctr + x;                  // next unclaimed item of this XCD's sequence

  uint32_t kofs[4], vofs;
  {
    const int r0 = 32 * wave + lane / CPR;
    const int pc = lane % CPR;
#pragma unroll
    for (int v = 0; v < 4; ++v) kofs[v] = static_cast<uint32_t>(r0 * 2 * D + 16 * (pc ^ swz_k<D>(r0 + RPI * v)));
    vofs = static_cast<uint32_t>(r0 * 2 * D + 16 * (pc ^ swz_v<D>(r0)));
  }
  // copies of tile kb of the K/V head that starts at kv (rows past the
  // sequence read as zeros, as in attn_fwd_kernel). Copy instruction i moves
  // RPI rows of 2D bytes = 1024 bytes further on in memory and in LDS, so its
  // immediate offset (added to both addresses) carries i % 4 and one LDS base
  // serves four instructions. The immediate field holds 12 bits (offsets past
  // 4095 do not encode), so instructions 4..7 take a second base 4096 bytes on.
  auto issue_k = [&](const uint16_t* kv, int kb) {
    const int key0 = kb * kBlock;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kv + static_cast<size_t>(key0) * D), 0,
                                                      (p.S - key0) * 2 * D, kBufferWord3);
    char* dst = reinterpret_cast<char*>(Ks) + 32 * wave * D * 2;
    static_for<NDMA>([&](auto I) {
      constexpr int i = decltype(I)::value, hi = i / 4;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + 4096 * hi), 16,
                                               (D == 128 ? kofs[i & 3] : kofs[0]) + 4096 * hi, 0, 1024 * (i % 4), 0);
    });
  };
  auto issue_v = [&](const uint16_t* kv, int kb) {
    const int key0 = kb * kBlock;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kv + static_cast<size_t>(key0) * D), 0,
                                                      (p.S - key0) * 2 * D, kBufferWord3);
    char* dst = reinterpret_cast<char*>(Vs) + 32 * wave * D * 2;
    static_for<NDMA>([&](auto I) {
      constexpr int i = decltype(I)::value, hi = i / 4;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + 4096 * hi), 16, vofs + 4096 * hi, 0,
                                               1024 * (i % 4), 0);
    });
  };
  uint32_t kaddr[KS], vaddr[MT];
  {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kaddr[ks] = lds_addr(Ks) + l32 * 2 * D + 16 * ((2 * ks + hl) ^ swz_k<D>(l32));
    const int G = lane >> 4, jj = (lane >> 2) & 3, a = lane & 3;
    const int key = 4 * (G >> 1) + jj;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      vaddr[mt] = lds_addr(Vs) + key * 2 * D + 16 * ((4 * mt + 2 * (G & 1) + (a >> 1)) ^ swz_v<D>(key)) + 8 * (a & 1);
  }

  // this lane's mask bytes of an item's chunk: keys c0 + lane and c0 + 64 +
  // lane (0 past the causal end, the diagonal included)
  auto load_flags = [&](const XcdItem& it, uint32_t& f0, uint32_t& f1) {
    f0 = 0;
    f1 = 0;
    if (it.bh < 0) return;
    const int c0 = it.c * kXcdDefaultChunk;
    const int kend = min(it.qb + 1, c0 + kXcdDefaultChunk);
    const uint8_t* mrow = p.mask + (static_cast<size_t>(it.bh) * p.nb + it.qb) * p.nb;
    if (c0 + lane < kend) f0 = mrow[c0 + lane];
    if (c0 + 64 + lane < kend) f1 = mrow[c0 + 64 + lane];
  };
  // Q rows of an item (rows past the sequence repeat the last one: their
  // outputs are never stored), as buffer loads: one scalar resource per item
  // and 32-bit lane offsets
  auto load_q = [&](const XcdItem& it, uint4 (&qr)[KS]) {
    const int t0 = it.qb * kBlock;
    const int t = min(t0 + q_local, p.S - 1);
    uint16_t* qblk = const_cast<uint16_t*>(p.q + (static_cast<size_t>(it.bh) * p.hs + t0) * D);
    const auto rq = __builtin_amdgcn_make_buffer_rsrc(qblk, 0, kBlock * D * 2, kBufferWord3);
    const uint32_t off = static_cast<uint32_t>(((t - t0) * D + 8 * hl) * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qr[ks] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, off + 32 * ks, 0, 0));
  };
  // first tile of an item: the diagonal if it is active, else the lowest active block
  auto first_tile = [&](const XcdItem& it, uint64_t f0, uint64_t f1) -> int {
    const int c0 = it.c * kXcdDefaultChunk;
    const int d = it.qb - c0;
    if (d < kXcdDefaultChunk && ((d < 64 ? (f0 >> d) : (f1 >> (d - 64))) & 1)) return it.qb;
    if (f0) return c0 + static_cast<int>(__builtin_ctzll(f0));
    if (f1) return c0 + 64 + static_cast<int>(__builtin_ctzll(f1));
    return -1;
  };

  // next active block of the item (ascending), -1 when none is left
  auto pop_flag = [](uint64_t& f0, uint64_t& f1, int c0) -> int {
    if (f0) {
      const int b = static_cast<int>(__builtin_ctzll(f0));
      f0 &= f0 - 1;
      return c0 + b;
    }
    if (f1) {
      const int b = static_cast<int>(__builtin_ctzll(f1));
      f1 &= f1 - 1;
      return c0 + 64 + b;
    }
    return -1;
  };

  // the first three items in one claim; afterwards one claim per item, two
  // items ahead (wave 0 lane 0 claims, LDS hands the index to both waves)
  __shared__ int claim;
  if (tid == 0) claim = atomicAdd(ctr, 3);
  __syncthreads();
  const int j0 = claim;
  XcdCursor cur;
  XcdItem it = xcd_item<D, kDiagPhase>(p, x, j0, cur);            // this item
  if (it.bh < 0) return;
  XcdItem it1 = xcd_item<D, kDiagPhase>(p, x, j0 + 1, cur);       // the next one
  int j2 = j0 + 2;                                 // the one after
  int pend = 0;                                    // wave 0 lane 0: claim in flight (the item after j2)
  bool claimed = false;

  const float c = p.scale_log2;
  uint4 qreg[KS];
  float m = -INFINITY, lsum = 0.f;
  f32x16_t oacc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) oacc[i] = f32x16_t{};

  // One tile kb_t of the K/V head at kvo_t; its K copies were issued before.
  // Two workgroup barriers per tile: the one that publishes K(t) also frees
  // the V buffer (both waves have read V(t-1)), so V(t) is copied from there
  // on; the one that publishes V(t) frees the K buffer, so the next tile's K
  // (`next` of the head at `nkv`; -1: none) is copied from there on. Each
  // batch of copies is issued while the wave's operand reads from LDS are in
  // flight, which hides the time the copy instructions take to issue. `qn`:
  // load the next item's Q rows into qreg once this tile's scores are issued.
  // `first`: the item's first tile (the only one that can be the diagonal),
  // which sets the running max; later tiles take their maximum only when it
  // could move it (tile_update_lazy).
  auto compute = [&](auto first_tag, bool diag, size_t kvo_t, int kb_t, size_t nkv, int next, bool qn) {
    constexpr bool first = decltype(first_tag)::value;
    wait_vm(0);                                    // this tile's K landed (and everything before it)
    wg_barrier();
    u32x4_t kr[2 * KS];
    read_k_issue<D>(kaddr, kr);
    issue_v(p.v + kvo_t, kb_t);
    read_k_wait<D>(kr);
    f32x16_t sacc[2];
    uint4 pb[4];
    if constexpr (first) {
      const float mx = tile_scores_rt<D>(kr, qreg, sacc, q_local, hl, c, diag);
      if (qn) load_q(it1, qreg);                   // qreg is free once the scores are issued
      tile_softmax_first(sacc, mx, c, m, lsum, pb);
    } else {
      tile_qk<D>(kr, qreg, sacc);
      if (qn) load_q(it1, qreg);
      tile_softmax_lazy<D>(sacc, c, m, lsum, oacc, pb);
    }
    wait_vm(qn ? KS : 0);                          // this tile's V landed
    wg_barrier();
    u32x2_t vr[8 * MT];
    read_v_issue<D>(vaddr, vr);
    if (next >= 0) issue_k(p.k + nkv, next);
    read_v_wait<D>(vr);
    tile_pv<D>(vr, pb, oacc);
  };

  // ---- prologue: the first item is started cold ---------------------------
  uint32_t fa0, fa1, fb0, fb1;                     // mask bytes: this item, the next one
  load_flags(it, fa0, fa1);
  load_flags(it1, fb0, fb1);
  wait_vm(0);
  uint64_t f0 = __builtin_amdgcn_ballot_w64(fa0 != 0), f1 = __builtin_amdgcn_ballot_w64(fa1 != 0);
  bool warm = false;                               // the item's Q and first K tile were issued during the previous one

  while (true) {
    // ---- item start ------------------------------------------------------
    const int c0 = it.c * kXcdDefaultChunk;
    const size_t kvo = static_cast<size_t>(it.kvo);
    int kb = first_tile(it, f0, f1);
    if (kb >= 0) {
      const int d = kb - c0;
      if (d < 64) f0 &= ~(1ull << d);
      else f1 &= ~(1ull << (d - 64));
    }
    if (!warm) {
      load_q(it, qreg);
      if (kb >= 0) issue_k(p.k + kvo, kb);
    }
    wait_vm(0);                                    // everything issued so far has landed
    const uint64_t g0 = __builtin_amdgcn_ballot_w64(fb0 != 0), g1 = __builtin_amdgcn_ballot_w64(fb1 != 0);
    if (claimed) {                                 // the claim issued at the previous item's start
      if (tid == 0) claim = pend;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      wg_barrier();
      j2 = __builtin_amdgcn_readfirstlane(static_cast<int>(lds_read_u32(lds_addr(&claim))));
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      wg_barrier();                                // both waves hold it before the LDS word is reused
    }
    const XcdItem it2 = xcd_item<D, kDiagPhase>(p, x, j2, cur);
    load_flags(it2, fb0, fb1);                     // the item after next; read at the next item's start
    claimed = it2.bh >= 0;
    if (claimed && tid == 0) {
      // an address the compiler cannot prove uniform: a uniform one makes it
      // read the result back at once (a wait for the atomic's round trip
      // here); this way the result is waited for only where it is used
      int off = 0;
      asm volatile("" : "+v"(off));
      pend = atomicAdd(ctr + off, 1);
    }
    const int kb1 = it1.bh >= 0 ? first_tile(it1, g0, g1) : -1;
    const size_t kvo1 = static_cast<size_t>(it1.kvo);

    // ---- tiles: the diagonal first, then ascending; the last one hands over
    // to the next item (its first tile's copies and its Q rows)
    warm = false;
    if (kb >= 0) {
      const bool diag = kb == it.qb;
      int next = pop_flag(f0, f1, c0);
      warm = it1.bh >= 0;
      if (next < 0) {
        compute(std::true_type{}, diag, kvo, kb, warm ? kvo1 : kvo, warm ? kb1 : -1, warm);
      } else {
        compute(std::true_type{}, diag, kvo, kb, kvo, next, false);
        int cur_kb = next;
        next = pop_flag(f0, f1, c0);
        while (next >= 0) {
          compute(std::false_type{}, false, kvo, cur_kb, kvo, next, false);
          cur_kb = next;
          next = pop_flag(f0, f1, c0);
        }
        compute(std::false_type{}, false, kvo, cur_kb, warm ? kvo1 : kvo, warm ? kb1 : -1, warm);
      }
    }

    // ---- epilogue ----------------------------------------------------------
    const float ltot = pair_sum(lsum);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    const float lse2 = ltot > 0.f ? m + __log2f(ltot) : -INFINITY;
    if constexpr (kDiagPhase) {
      // the row's last chunk: merged with its earlier chunks' partials
      float inv_r = inv, lse2_r = lse2;
      if (it.c > 0) merge_chunk_partials<D, 3>(p, it.bh, it.qb, it.c, tid, q_local, oacc, inv_r, lse2_r);
      const int t = it.qb * kBlock + q_local;
      if (t < p.S) {
        const size_t obase = (static_cast<size_t>(it.bh) * p.hs + t) * D;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int dim = 32 * mt + 8 * r4 + 4 * hl;
            const float o0 = oacc[mt][4 * r4 + 0] * inv_r, o1 = oacc[mt][4 * r4 + 1] * inv_r;
            const float o2 = oacc[mt][4 * r4 + 2] * inv_r, o3 = oacc[mt][4 * r4 + 3] * inv_r;
            if (p.out_bf16) {
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + obase + dim) =
                  make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
            } else {
              *reinterpret_cast<float4*>(static_cast<float*>(p.out) + obase + dim) = make_float4(o0, o1, o2, o3);
            }
          }
        }
        if (p.lse != nullptr && hl == 0) p.lse[static_cast<size_t>(it.bh) * p.hs + t] = lse2_r * kLn2;
      }
    } else {
      // normalized bf16 partial: the thread's 8-value group g (oacc[g / 2]
      // values 8 (g % 2) ..) is 16 bytes at uint4 index g * kThreads + tid of
      // the slot, so each store instruction writes 1 KiB contiguous. The
      // stores are non-temporal: the partials are read once, by the merge, and
      // would otherwise push the chunk's K/V out of the XCD's L2
      const long long slot = static_cast<long long>(it.bh) * p.slots_per_head +
                             xcd_slot_base(it.qb, kXcdDefaultChunk) + it.c;
      uint4* po = reinterpret_cast<uint4*>(p.part_o16 + slot * kBlock * D) + tid;
  #pragma unroll
      for (int mt = 0; mt < MT; ++mt)
  #pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
          __builtin_nontemporal_store(
              u32x4_t{pack_bf16x2(oacc[mt][8 * h2 + 0] * inv, oacc[mt][8 * h2 + 1] * inv),
                      pack_bf16x2(oacc[mt][8 * h2 + 2] * inv, oacc[mt][8 * h2 + 3] * inv),
                      pack_bf16x2(oacc[mt][8 * h2 + 4] * inv, oacc[mt][8 * h2 + 5] * inv),
                      pack_bf16x2(oacc[mt][8 * h2 + 6] * inv, oacc[mt][8 * h2 + 7] * inv)},
              reinterpret_cast<u32x4_t*>(po + (2 * mt + h2) * kThreads));
      if (hl == 0) p.part_l[slot * kBlock + q_local] = lse2;
    }
    m = -INFINITY;
    lsum = 0.f;
#pragma unroll
    for (int i = 0; i < MT; ++i) oacc[i] = f32x16_t{};

    if (it1.bh < 0) break;
    it = it1;
    it1 = it2;
    f0 = g0;
    f1 = g1;
  }
}

// Per-XCD item counters of attn_sparse_xcd_kernel start at 0 on every call.
__global__ void attn_xcd_counters_init(int* ctr) {
  if (threadIdx.x < kXcds) ctr[threadIdx.x] = 0;
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
  if (mode == kSparse && a.xcd) {
    hipLaunchKernelGGL(attn_xcd_counters_init, dim3(1), dim3(kWave), 0, st, a.xcd_ctr);
    hipLaunchKernelGGL((attn_sparse_xcd_kernel<D, false>), dim3(kXcds * kXcdSlots), block, 0, st, a);
    hipLaunchKernelGGL(attn_xcd_counters_init, dim3(1), dim3(kWave), 0, st, a.xcd_ctr);
    hipLaunchKernelGGL((attn_sparse_xcd_kernel<D, true>), dim3(kXcds * kXcdSlots), block, 0, st, a);
    return hipGetLastError();
  }
  if constexpr (D == 128) {
    if (mode == kSparse && a.rows) {
      hipLaunchKernelGGL(attn_rows_counters_init, dim3(1), dim3(kWave), 0, st, a.xcd_ctr);
      hipLaunchKernelGGL((attn_sparse_rows_kernel<D>), dim3(kXcds * kRowSlots), block, 0, st, a);
      return hipGetLastError();
    }
  }
  if (mode == kSparse) {
    if (a.xcd_work != nullptr) {
      hipLaunchKernelGGL(attn_xcd_counters_init, dim3(1), dim3(kWave), 0, st, a.xcd_work);
      const dim3 wgrid(static_cast<unsigned>(a.B) * a.Hq, static_cast<unsigned>((a.nb + kWorkRows - 1) / kWorkRows));
      hipLaunchKernelGGL(attn_xcd_work_kernel, wgrid, dim3(256), 0, st, a);
    }
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
  if (a.group % kGqaHeads == 0) {
    // the query heads of a KV group four at a time, sharing K/V tile copies
    const dim3 grid(static_cast<unsigned>(a.B) * a.Hq / kGqaHeads * a.nb), gblock(kGqaThreads);
    if (mode == kDense) hipLaunchKernelGGL((attn_dense_gqa_kernel<D, kDense>), grid, gblock, 0, st, a);
    else hipLaunchKernelGGL((attn_dense_gqa_kernel<D, kDenseGt>), grid, gblock, 0, st, a);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>(a.B) * a.Hq * a.nb);
  if (mode == kDense) hipLaunchKernelGGL((attn_fwd_kernel<D, kDense>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((attn_fwd_kernel<D, kDenseGt>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

namespace {
// Key blocks per chunk of the other block-sparse path: up to 1024 blocks (64k
// tokens) a row is one item; longer rows are cut into chunks of 512 blocks,
// which the XCDs sweep together.
int sweep_chunk_blocks(int nb) { return nb > 1024 ? 512 : kListCap; }
constexpr long long kXcdRowsMaxBlockDims = 256 * 128;   // key blocks x head_dim
}  // namespace

// The XCD-owned path takes rows of at least kXcdMinBlocks blocks when there
// are at least 64 (batch, KV group, chunk) jobs to deal over the 8 XCDs (with
// 32/8 heads at 90% it measured 4% faster than the persistent rows at 60k and
// 12% at 64k, 3-8% slower at 48k and 56k, where fewer K/V re-reads miss the
// L2); otherwise the rows go to attn_sparse_rows_kernel or attn_fwd_kernel
// (cut into chunks of 512 blocks above 1024 blocks, with the circular sweep).
SparsePlan sparse_plan(int B, int Hkv, int group, int nb, int D) {
  SparsePlan pl{};
  const int C = kXcdDefaultChunk;
  const long long nch = (nb + C - 1) / C;
  const long long jobs = static_cast<long long>(B) * Hkv * nch;
  pl.xcd = nb >= kXcdMinBlocks && jobs >= 64;
  if (pl.xcd) {
    pl.chunk = C;                                  // attn_sparse_xcd_kernel assumes this chunk size
    pl.nchunk = static_cast<int>(nch);
    pl.njobs = static_cast<int>(jobs);
    pl.slots_per_head = xcd_slot_base(nb, C);
    const size_t slots = static_cast<size_t>(B) * Hkv * group * pl.slots_per_head;
    pl.workspace_bytes = slots * kBlock * (static_cast<size_t>(D) * sizeof(uint16_t) + sizeof(float)) + 256;
    return pl;
  }
  pl.chunk = sweep_chunk_blocks(nb);
  pl.nchunk = (nb + pl.chunk - 1) / pl.chunk;
  pl.rotate = 1;
  // the XCD-major order of one-item rows, for rows of up to 256 blocks at
  // D = 128 (512 at D = 64: K and V of a KV head up to twice an XCD's L2),
  // where it measured faster on balanced masks, and heads that split evenly
  // over the 8 XCDs; 256 bytes of per-XCD counts
  pl.xcd_rows = pl.nchunk == 1 && static_cast<long long>(nb) * D <= kXcdRowsMaxBlockDims &&
                (static_cast<long long>(B) * Hkv * group) % kXcds == 0;
  // longer one-item rows at D = 128 with at least 8 rows per resident
  // workgroup: the persistent launch of attn_sparse_rows_kernel, 256 bytes of
  // per-queue counters
  pl.rows = pl.nchunk == 1 && D == 128 && static_cast<long long>(nb) * D > kXcdRowsMaxBlockDims &&
            static_cast<long long>(B) * Hkv * group * nb >= 8LL * kXcds * kRowSlots;
  const long long nc = pl.nchunk;
  pl.items_per_group = static_cast<long long>(group) * (nc * nb - static_cast<long long>(pl.chunk) * nc * (nc - 1) / 2);
  if (nb > pl.chunk) {
    const size_t items = static_cast<size_t>(B) * Hkv * pl.items_per_group;
    pl.workspace_bytes = items * kBlock * (static_cast<size_t>(D) + 1) * sizeof(float);
  } else if (pl.xcd_rows || pl.rows) {
    pl.workspace_bytes = 256;
  }
  return pl;
}

hipError_t launch_attn(const AttnArgs& a, int mode, hipStream_t st) {
  if (a.D == 64) return launch_d<64>(a, mode, st);
  return launch_d<128>(a, mode, st);
}

int varlen_chunk_blocks() { return kListCap; }

hipError_t launch_attn_varlen(const AttnArgs& a, const VarlenTable& t, int mode, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(t.row_start[t.n])), block(kThreads);
  if (a.D == 64) {
    if (mode == kSparse) hipLaunchKernelGGL((attn_varlen_kernel<64, kSparse>), grid, block, 0, st, a, t);
    else if (mode == kDense) hipLaunchKernelGGL((attn_varlen_kernel<64, kDense>), grid, block, 0, st, a, t);
    else hipLaunchKernelGGL((attn_varlen_kernel<64, kDenseGt>), grid, block, 0, st, a, t);
  } else {
    if (mode == kSparse) hipLaunchKernelGGL((attn_varlen_kernel<128, kSparse>), grid, block, 0, st, a, t);
    else if (mode == kDense) hipLaunchKernelGGL((attn_varlen_kernel<128, kDense>), grid, block, 0, st, a, t);
    else hipLaunchKernelGGL((attn_varlen_kernel<128, kDenseGt>), grid, block, 0, st, a, t);
  }
  return hipGetLastError();
}

}  // namespace seer
