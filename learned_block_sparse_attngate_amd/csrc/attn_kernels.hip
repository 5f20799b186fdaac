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
constexpr int kSweepPhases = 128;        // resident workgroups per XCD (32 CUs x 4)

enum Mode { kSparse = 0, kDense = 1, kDenseGt = 2 };


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
    wait_vm(first ? NDMA : NDMA + stores_pending);
    wg_barrier();
    u32x4_t kr[2 * KS];                           // kr[2 ks + mt]: keys 32 mt + l32, dims 16 ks + 8 hl ..
    read_k_tile<D>(kaddr, kr);
    wg_barrier();                                  // both waves hold K: refill the K buffer
    if (next >= 0) issue_k(next);

    f32x16_t sacc[2];
    float mx = tile_scores<D, kDiag>(kr, qreg, sacc, q_local, hl, c);
    int stores_now = 0;
    if constexpr (MODE == kDenseGt) {
      if (hl == 0) p.rmax[((static_cast<size_t>(bh) * p.ntri + ntri_off + kb) << 6) + q_local] = mx;
      stores_now = 1;
    }

    // ---- V: wait for the copy (the K copy of `next` and this tile's store may be newer)
    wait_vm((next >= 0 ? NDMA : 0) + stores_now);
    wg_barrier();
    u32x2_t vr[8 * MT];                            // vr[(ks MT + mt) 2 + u]: dims 32 mt + .., keys 16 ks + 8 u + ..
    read_v_tile<D>(vaddr, vr);
    wg_barrier();                                  // both waves hold V: refill the V buffer
    if (next >= 0) issue_v(next);
    stores_pending = stores_now;

    tile_update<D>(sacc, vr, mx, c, m, lsum, oacc);
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
      wait_vm(0);                            // the early copy of the diagonal tile is not used
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

// ---------------------------------------------------------------------------
// Block-sparse rows of many key blocks: XCD-owned key chunks, persistent
// workgroups.
//
// The key range is cut into chunks of C blocks. A job is one chunk of one
// (batch, KV group): the (row, chunk) items of every query head of the group
// whose causal range reaches the chunk, head major, query block descending.
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
// ahead, the next item's mask flags one item ahead, and its Q rows and first
// K/V tile are issued during the current item's last tile. An item of a row
// that spans several chunks writes a bf16 partial output (normalized by its
// own sum) and its log2-sum-exp; attn_xcd_combine_kernel merges them. Rows
// inside the first chunk are one item and are written directly.
constexpr int kXcdMaxChunk = 128;        // key blocks per chunk at most (two 64-bit flag words)
constexpr int kXcdDefaultChunk = 128;    // 4 MiB of K/V at D = 128: one XCD's L2
constexpr int kXcdMinBlocks = 1280;      // rows of 80k tokens and more
constexpr int kXcdSlots = 128;           // resident workgroups per XCD: 32 CUs x 4


// Job at position t of XCD x's sequence, or -1 past its end. Positions 2i and
// 2i+1 take jobs 16i + x and 16i + 15 - x; the first job past the end ends it.
__device__ __forceinline__ int xcd_job(int x, int t, int njobs) {
  const int base = 2 * kXcds * (t >> 1);
  const int k = (t & 1) ? base + 2 * kXcds - 1 - x : base + x;
  return k < njobs ? k : -1;
}

struct XcdItem {
  int bh;      // batch * Hq + head; -1: past the end of the sequence
  int qb;      // query block
  int c;       // key chunk
};

// Walks one XCD's item sequence; queried with increasing item indices (the
// host keeps every index within 32 bits).
struct XcdCursor {
  int t = 0;
  int job = -1;
  int begin = 0;           // sequence index of the job's first item
  int count = 0;           // items in the job
};

__device__ __forceinline__ XcdItem xcd_item(const AttnArgs& p, int x, int j, XcdCursor& cur) {
  while (true) {
    if (cur.job < 0) {
      cur.job = xcd_job(x, cur.t, p.njobs);
      if (cur.job < 0) return XcdItem{-1, 0, 0};
      cur.count = p.group * (p.nb - (cur.job % p.nchunk) * p.chunk);
    }
    if (j < cur.begin + cur.count) break;
    cur.begin += cur.count;
    ++cur.t;
    cur.job = -1;
  }
  const int c = cur.job % p.nchunk, gi = cur.job / p.nchunk;
  const int rows = p.nb - c * p.chunk;
  const int mi = j - cur.begin;
  const int hig = mi / rows;
  const int bb = gi / p.Hkv, gg = gi - bb * p.Hkv;
  return XcdItem{bb * p.Hq + gg * p.group + hig, p.nb - 1 - (mi - hig * rows), c};
}

// Partial-output slots before query block qb of one head: rows qb' >= C own
// qb'/C + 1 slots each (one per key chunk they reach).
__device__ __host__ __forceinline__ long long xcd_slot_base(long long qb, long long C) {
  const long long k = qb / C;
  return qb + C * k * (k - 1) / 2 + k * (qb - k * C) - C;
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_sparse_xcd_kernel(AttnArgs p) {
  constexpr int CPR = D / 8;               // 16-byte chunks per K/V row
  constexpr int KS = D / 16;               // MFMA k-steps for S^T (= Q loads per thread)
  constexpr int MT = D / 32;               // MFMA m-tiles for O^T
  constexpr int RPI = 64 / CPR;            // tile rows per copy instruction
  constexpr int NDMA = 32 / RPI;           // copy instructions per wave per operand
  constexpr int HALF = D / 2;              // output values per thread

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

  auto kv_head = [&](const XcdItem& it) -> size_t {
    const int b = it.bh / p.Hq;
    const int g = (it.bh - b * p.Hq) / p.group;
    return (static_cast<size_t>(b) * p.Hkv + g) * p.hs * D;
  };
  // this lane's mask bytes of an item's chunk: keys c0 + lane and c0 + 64 +
  // lane (0 past the causal end, the diagonal included)
  auto load_flags = [&](const XcdItem& it, uint32_t& f0, uint32_t& f1) {
    f0 = 0;
    f1 = 0;
    if (it.bh < 0) return;
    const int c0 = it.c * p.chunk;
    const int kend = min(it.qb + 1, c0 + p.chunk);
    const uint8_t* mrow = p.mask + (static_cast<size_t>(it.bh) * p.nb + it.qb) * p.nb;
    if (c0 + lane < kend) f0 = mrow[c0 + lane];
    if (c0 + 64 + lane < kend) f1 = mrow[c0 + 64 + lane];
  };
  // Q rows of an item (rows past the sequence repeat the last one: their
  // outputs are never stored)
  auto load_q = [&](const XcdItem& it, uint4 (&qr)[KS]) {
    const int t = min(it.qb * kBlock + q_local, p.S - 1);
    const uint16_t* qrow = p.q + (static_cast<size_t>(it.bh) * p.hs + t) * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qr[ks] = *reinterpret_cast<const uint4*>(qrow + 16 * ks);
  };
  // first tile of an item: the diagonal if it is active, else the lowest active block
  auto first_tile = [&](const XcdItem& it, uint64_t f0, uint64_t f1) -> int {
    const int c0 = it.c * p.chunk;
    const int d = it.qb - c0;
    if (d < p.chunk && ((d < 64 ? (f0 >> d) : (f1 >> (d - 64))) & 1)) return it.qb;
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
  XcdItem it = xcd_item(p, x, j0, cur);            // this item
  if (it.bh < 0) return;
  XcdItem it1 = xcd_item(p, x, j0 + 1, cur);       // the next one
  int j2 = j0 + 2;                                 // the one after
  int pend = 0;                                    // wave 0 lane 0: claim in flight (the item after j2)
  bool claimed = false;

  const float c = p.scale_log2;
  uint4 qreg[KS];
  float m = -INFINITY, lsum = 0.f;
  f32x16_t oacc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) oacc[i] = f32x16_t{};

  // One tile; its copies were issued before. `tile0`: the item's first tile,
  // whose copies (and everything else issued earlier) have landed. `nkv`:
  // offset of the K/V head of the next tile `next` (-1: none). `qn`: load the
  // next item's Q rows into qreg once this tile's scores are computed.
  auto compute = [&](bool diag, bool tile0, size_t nkv, int next, bool qn) {
    if (!tile0) wait_vm(NDMA);                     // this tile's K landed (its V may be in flight)
    wg_barrier();
    u32x4_t kr[2 * KS];
    read_k_tile<D>(kaddr, kr);
    wg_barrier();                                  // both waves hold K: refill the K buffer
    if (next >= 0) issue_k(p.k + nkv, next);
    f32x16_t sacc[2];
    const float mx = tile_scores_rt<D>(kr, qreg, sacc, q_local, hl, c, diag);
    if (qn) load_q(it1, qreg);                     // qreg is free once the scores are issued
    if (!tile0) wait_vm((next >= 0 ? NDMA : 0) + (qn ? KS : 0));   // this tile's V landed
    wg_barrier();
    u32x2_t vr[8 * MT];
    read_v_tile<D>(vaddr, vr);
    wg_barrier();                                  // both waves hold V: refill the V buffer
    if (next >= 0) issue_v(p.v + nkv, next);
    tile_update<D>(sacc, vr, mx, c, m, lsum, oacc);
  };

  // ---- prologue: the first item is started cold ---------------------------
  uint32_t fa0, fa1, fb0, fb1;                     // mask bytes: this item, the next one
  load_flags(it, fa0, fa1);
  load_flags(it1, fb0, fb1);
  wait_vm(0);
  uint64_t f0 = __builtin_amdgcn_ballot_w64(fa0 != 0), f1 = __builtin_amdgcn_ballot_w64(fa1 != 0);
  bool warm = false;                               // the item's Q and first tile were issued during the previous one

  while (true) {
    // ---- item start ------------------------------------------------------
    const int c0 = it.c * p.chunk;
    const size_t kvo = kv_head(it);
    int kb = first_tile(it, f0, f1);
    if (kb >= 0) {
      const int d = kb - c0;
      if (d < 64) f0 &= ~(1ull << d);
      else f1 &= ~(1ull << (d - 64));
    }
    if (!warm) {
      load_q(it, qreg);
      if (kb >= 0) {
        issue_k(p.k + kvo, kb);
        issue_v(p.v + kvo, kb);
      }
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
    const XcdItem it2 = xcd_item(p, x, j2, cur);
    load_flags(it2, fb0, fb1);                     // the item after next; read at the next item's start
    claimed = it2.bh >= 0;
    if (claimed && tid == 0) pend = atomicAdd(ctr, 1);
    const int kb1 = it1.bh >= 0 ? first_tile(it1, g0, g1) : -1;
    const size_t kvo1 = it1.bh >= 0 ? kv_head(it1) : 0;

    // ---- tiles: the diagonal first, then ascending; the last one hands over
    // to the next item (its first tile's copies and its Q rows)
    warm = false;
    if (kb >= 0) {
      bool tile0 = true;
      bool diag = kb == it.qb;
      int next = pop_flag(f0, f1, c0);
      while (next >= 0) {
        compute(diag, tile0, kvo, next, false);
        tile0 = false;
        diag = false;
        next = pop_flag(f0, f1, c0);
      }
      warm = it1.bh >= 0;
      compute(diag, tile0, warm ? kvo1 : kvo, warm ? kb1 : -1, warm);
    }

    // ---- epilogue ----------------------------------------------------------
    const float ltot = pair_sum(lsum);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    const float lse2 = ltot > 0.f ? m + __log2f(ltot) : -INFINITY;
    if (it.qb >= p.chunk) {
      // normalized bf16 partial: the thread's 8-value group g (oacc[g / 2]
      // values 8 (g % 2) ..) is 16 bytes at uint4 index g * kThreads + tid of
      // the slot, so each store instruction writes 1 KiB contiguous
      const long long slot = static_cast<long long>(it.bh) * p.slots_per_head +
                             xcd_slot_base(it.qb, p.chunk) + it.c;
      uint4* po = reinterpret_cast<uint4*>(p.part_o16 + slot * kBlock * D) + tid;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
          po[(2 * mt + h2) * kThreads] =
              make_uint4(pack_bf16x2(oacc[mt][8 * h2 + 0] * inv, oacc[mt][8 * h2 + 1] * inv),
                         pack_bf16x2(oacc[mt][8 * h2 + 2] * inv, oacc[mt][8 * h2 + 3] * inv),
                         pack_bf16x2(oacc[mt][8 * h2 + 4] * inv, oacc[mt][8 * h2 + 5] * inv),
                         pack_bf16x2(oacc[mt][8 * h2 + 6] * inv, oacc[mt][8 * h2 + 7] * inv));
      if (hl == 0) p.part_l[slot * kBlock + q_local] = lse2;
    } else {
      const int t = it.qb * kBlock + q_local;
      if (t < p.S) {
        const size_t obase = (static_cast<size_t>(it.bh) * p.hs + t) * D;
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
        if (p.lse != nullptr && hl == 0) p.lse[static_cast<size_t>(it.bh) * p.hs + t] = lse2 * kLn2;
      }
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

// Merge of the bf16 partials written by attn_sparse_xcd_kernel:
// O = sum_c w_c O_c / sum_c w_c, w_c = 2^(L_c - max L), LSE = max L + log2(sum w).
// One workgroup per row qb >= C, thread and value layout as in the writer. The slots are
// read kXcdMergeBatch at a time, all loads of a batch issued before any is
// used, so the merge runs at memory bandwidth rather than one latency per slot.
constexpr int kXcdMergeBatch = 4;

template <int D>
__global__ __launch_bounds__(kThreads) void attn_xcd_combine_kernel(AttnArgs p) {
  constexpr int MT = D / 32;
  constexpr int HALF = D / 2;
  constexpr int NV = HALF / 8;                     // 16-byte loads per thread and slot
  const int rows = p.nb - p.chunk;
  const int bh = blockIdx.x / rows;
  const int qb = p.chunk + static_cast<int>(blockIdx.x % rows);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int q_local = wave * 32 + l32;
  const int n = qb / p.chunk + 1;
  const long long slot0 = static_cast<long long>(bh) * p.slots_per_head + xcd_slot_base(qb, p.chunk);
  const float* lse = p.part_l + slot0 * kBlock + q_local;
  float lmax = -INFINITY;
  for (int c0 = 0; c0 < n; c0 += 2 * kXcdMergeBatch) {
    float l[2 * kXcdMergeBatch];
#pragma unroll
    for (int u = 0; u < 2 * kXcdMergeBatch; ++u) l[u] = c0 + u < n ? lse[(c0 + u) * kBlock] : -INFINITY;
#pragma unroll
    for (int u = 0; u < 2 * kXcdMergeBatch; ++u) lmax = fmaxf(lmax, l[u]);
  }
  float acc[HALF];
#pragma unroll
  for (int i = 0; i < HALF; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  if (lmax > -INFINITY) {
    const uint4* src = reinterpret_cast<const uint4*>(p.part_o16 + slot0 * kBlock * D) + tid;
    for (int c0 = 0; c0 < n; c0 += kXcdMergeBatch) {
      uint4 v[kXcdMergeBatch][NV];
      float w[kXcdMergeBatch];
#pragma unroll
      for (int u = 0; u < kXcdMergeBatch; ++u) {
        const bool ok = c0 + u < n;
        const int cc = ok ? c0 + u : c0;           // a slot that exists; its weight is 0 below
        w[u] = ok ? lse[cc * kBlock] : -INFINITY;
#pragma unroll
        for (int i = 0; i < NV; ++i) v[u][i] = src[static_cast<long long>(cc) * (kBlock * D / 8) + i * kThreads];
      }
#pragma unroll
      for (int u = 0; u < kXcdMergeBatch; ++u) {
        const float wu = __builtin_amdgcn_exp2f(w[u] - lmax);
        wsum += wu;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const uint32_t wd[4] = {v[u][i].x, v[u][i].y, v[u][i].z, v[u][i].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[8 * i + 2 * e] = fmaf(wu, __uint_as_float(wd[e] << 16), acc[8 * i + 2 * e]);
            acc[8 * i + 2 * e + 1] = fmaf(wu, __uint_as_float(wd[e] & 0xffff0000u), acc[8 * i + 2 * e + 1]);
          }
        }
      }
    }
  }
  const int t = qb * kBlock + q_local;
  if (t >= p.S) return;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const size_t obase = (static_cast<size_t>(bh) * p.hs + t) * D;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int dim = 32 * mt + 8 * r4 + 4 * hl;
      const float* a = acc + 16 * mt + 4 * r4;
      if (p.out_bf16) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + obase + dim) =
            make_uint2(pack_bf16x2(a[0] * inv, a[1] * inv), pack_bf16x2(a[2] * inv, a[3] * inv));
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + obase + dim) =
            make_float4(a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv);
      }
    }
  }
  if (p.lse != nullptr && hl == 0)
    p.lse[static_cast<size_t>(bh) * p.hs + t] = wsum > 0.f ? (lmax + __log2f(wsum)) * kLn2 : -INFINITY;
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
    hipLaunchKernelGGL((attn_sparse_xcd_kernel<D>), dim3(kXcds * kXcdSlots), block, 0, st, a);
    if (a.nb > a.chunk) {
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const dim3 cgrid(static_cast<unsigned>(a.B) * a.Hq * (a.nb - a.chunk));
      hipLaunchKernelGGL((attn_xcd_combine_kernel<D>), cgrid, block, 0, st, a);
    }
    return hipGetLastError();
  }
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

namespace {
// Key blocks per chunk of the other block-sparse path. Up to 1024 blocks (64k
// tokens) a row is one item; longer rows are cut into chunks of 512 blocks,
// which the XCDs sweep together. SEER_ATTN_CHUNK overrides the chunk (rounded
// to a multiple of 16, at most the on-chip list capacity).
int sweep_chunk_blocks(int nb) {
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
}  // namespace

// The XCD-owned path takes rows of at least kXcdMinBlocks blocks when there
// are at least 64 (batch, KV group, chunk) jobs to deal over the 8 XCDs (it
// measured 1-3% faster than the other path from 80k tokens up, slower at 64k
// and below, where fewer K/V re-reads miss the L2); otherwise the rows go to
// attn_fwd_kernel (cut into chunks of 512 blocks above 1024 blocks, with the
// circular sweep). SEER_ATTN_XCD=0 / 1 forces the choice (1: whenever rows
// reach a second chunk), SEER_XCD_CHUNK sets its chunk (16..128) and
// SEER_ATTN_ROTATE=0 turns the sweep off.
SparsePlan sparse_plan(int B, int Hkv, int group, int nb, int D) {
  static const int forced_xcd = [] {
    const char* v = getenv("SEER_ATTN_XCD");
    return v == nullptr ? -1 : (atoi(v) != 0);
  }();
  static const int forced_rotate = [] {
    const char* v = getenv("SEER_ATTN_ROTATE");
    return v == nullptr ? -1 : (atoi(v) != 0);
  }();
  static const int xcd_chunk = [] {
    const char* v = getenv("SEER_XCD_CHUNK");
    int x = v == nullptr ? kXcdDefaultChunk : atoi(v);
    return x < 16 ? 16 : (x > kXcdMaxChunk ? kXcdMaxChunk : x);
  }();
  SparsePlan pl{};
  const int C = xcd_chunk;
  const long long nch = (nb + C - 1) / C;
  const long long jobs = static_cast<long long>(B) * Hkv * nch;
  pl.xcd = forced_xcd >= 0 ? (forced_xcd && nb > C) : (nb >= kXcdMinBlocks && jobs >= 64);
  if (pl.xcd) {
    pl.chunk = C;
    pl.nchunk = static_cast<int>(nch);
    pl.njobs = static_cast<int>(jobs);
    pl.slots_per_head = xcd_slot_base(nb, C);
    const size_t slots = static_cast<size_t>(B) * Hkv * group * pl.slots_per_head;
    pl.workspace_bytes = slots * kBlock * (static_cast<size_t>(D) * sizeof(uint16_t) + sizeof(float)) + 256;
    return pl;
  }
  pl.chunk = sweep_chunk_blocks(nb);
  pl.nchunk = (nb + pl.chunk - 1) / pl.chunk;
  pl.rotate = forced_rotate >= 0 ? forced_rotate : 1;
  const long long nc = pl.nchunk;
  pl.items_per_group = static_cast<long long>(group) * (nc * nb - static_cast<long long>(pl.chunk) * nc * (nc - 1) / 2);
  if (nb > pl.chunk) {
    const size_t items = static_cast<size_t>(B) * Hkv * pl.items_per_group;
    pl.workspace_bytes = items * kBlock * (static_cast<size_t>(D) + 1) * sizeof(float);
  }
  return pl;
}

hipError_t launch_attn(const AttnArgs& a, int mode, hipStream_t st) {
  if (a.D == 64) return launch_d<64>(a, mode, st);
  return launch_d<128>(a, mode, st);
}

}  // namespace seer
