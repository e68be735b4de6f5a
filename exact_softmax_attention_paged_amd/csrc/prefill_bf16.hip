// Prefill attention kernel, bf16 in / fp32 accumulate, for gfx950.
//
// Method (vLLM FlashAttention page, sections "들어가며" and "논문 핵심 내용"): Q, K and V are
// brought on chip tile by tile, the softmax is carried online with a running max and a running
// sum, and only the final rows (plus their log-sum-exp) are written, so no score matrix ever
// reaches HBM. K/V rows are read through the block table from the paged cache of the
// FlashAttentionBackend section; GQA follows num_queries_per_kv of the FlashAttentionImpl
// section; causal and sliding-window masks follow the RBLN "Attention 모드" page.
//
// Work split: one workgroup = 8 waves of one (request, q head); each wave owns 32 query rows,
// one 32-wide MFMA column block, so a workgroup covers 256 rows and every K/V tile brought on
// chip serves 256 queries. KV is walked in tiles (128 keys for d = 128, 64 for d = 64)
// through two LDS buffers:
//   * the next tile's K and V rows go from HBM straight into the other buffer
//     (global_load_lds_dwordx4) while the current tile is consumed: no register staging and
//     no LDS stores. Every wave issues its share of them between its QK^T k-chunks. The
//     block ids of the tile after it are fetched at the same time, so the addresses are
//     ready when its loads are issued; one barrier per tile;
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 (K from LDS as the A operand, Q^T held in
//     registers as the B operand). On gfx950 this shape sustains about 1.6x the bf16 rate of
//     the 16x16x32 shape. Each lane holds 16 keys of one query, so the row max and row sum
//     need one v_permlane32_swap;
//   * P^T stays in registers and is already in the B-operand layout of the PV MFMA;
//   * O^T += V^T . P^T, with V^T read straight from the row-major V tile by
//     ds_read_b64_tr_b16, so no transpose pass is needed;
//   * each lane owns one query column of O^T, so the softmax rescale is lane-local. The
//     reference max is only moved when a new score exceeds it by more than 2^8 (in exp2
//     units): the result O / l is the same for any reference, the skipped rescales save most
//     of the per-tile VALU work, and p = 2^(s*c - m*c) stays <= 256.
//
// v_mfma_f32_32x32x16_bf16 lane layout (lane l, h = l / 32), checked on gfx950:
//   A (32 x 16): element e of lane l is A[l % 32][8h + e]
//   B (16 x 32): element e of lane l is B[8h + e][l % 32]
//   C (32 x 32): element e of lane l is C[8(e / 4) + 4h + e % 4][l % 32]
#include <algorithm>

#include "decode_core.hpp"
#include "device_common.hpp"
#include "kernels.hpp"

namespace attn {
namespace {

constexpr int kRows = 32;     // query rows per wave
constexpr float kRescaleLog2 = 8.f;
// Maximum of scores, which hold no NaN: IEEE maximum (v_maximum3_f32 on gfx950) needs no
// quieting of its operands, whereas fmaxf first canonicalises each MFMA result that it cannot
// prove canonical (one more v_max per operand).
__device__ __forceinline__ float max3_f32(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
__device__ __forceinline__ float max_f32(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

constexpr int kWaves = 8;                    // waves per workgroup (2 per SIMD)
// Keys per KV tile: 128 for d = 128 (half the per-tile overhead: barrier, row-max reduction,
// load issue), 64 for d = 64, whose short, ragged sequences waste more of a long tile
// (measured on gfx950: d 128 causal 994 -> 1040 TFLOP/s with 128; d 64 varlen 264 -> 216).
// The 128-key d = 128 kernel uses all 256 VGPRs with no spill.
template <int D>
constexpr int tile_keys() { return D == 128 ? 128 : 64; }
constexpr int kThreads = kWaves * kWave;
constexpr int kBR = kWaves * kRows;          // query rows per workgroup
constexpr int kBufs = 2;                     // LDS K/V buffers (prefetch distance 1)

typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ floatx16 mfma32x32x16(const bf16x8& a, const bf16x8& b,
                                                 const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS chunk permutation of K/V row r (16-byte chunks; 16 per row for d = 128, 8 for d = 64):
// the 16 rows read by one half-wave pass of the K operand hit 16 distinct bank groups, and
// the 4 rows x 4 chunks read by one pass of the transposing V reads are all distinct.
template <int D>
__device__ __forceinline__ int swizzle(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Wait for all of this wave's outstanding vector-memory operations (the direct global->LDS
// loads and the block-id loads of the next tile). gfx9 s_waitcnt: vmcnt 0, expcnt and lgkmcnt
// left alone.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier for the K/V buffers, called after wait_vmem(). The memory clobber keeps
// the compiler from moving memory operations across it; lgkmcnt(0) completes this wave's LDS
// reads of the tile before another wave may refill its buffer.
__device__ __forceinline__ void barrier_kv() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Transposing LDS read (ds_read_b64_tr_b16) at an LDS byte address.
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
__device__ __attribute__((always_inline)) inline bf16x4 tr_read(
    const lds_shortx4* __restrict__ ptr) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                        const_cast<lds_shortx4*>(ptr)));
}
// Direct load of 16 bytes per lane from global memory into LDS at lds_base + 16 * lane
// (global_load_lds_dwordx4, M0 = lds_base; s_nop covers the M0-write hazard). Issued as
// inline assembly so that the compiler's wait-count model sees no outstanding LDS write:
// with the intrinsic it waits for every LDS read (lgkmcnt(0)) before each MFMA operand use
// instead of only for the one it needs. Completion is waited for explicitly (wait_vmem
// before the tile barrier), and nothing else in these kernels uses M0.
__device__ __forceinline__ void dma_b128(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ const lds_shortx4* lds_at(uint32_t byte_addr) {
  return (const lds_shortx4*)(uintptr_t)byte_addr;
}

// Bytes of the K/V tile buffers of one workgroup.
template <int D>
constexpr int kv_lds_bytes() { return kBufs * 2 * tile_keys<D>() * 2 * D; }

// The work of one prefill workgroup: q tile and q head from the schedule slot bx / num_heads
// (scheduled launches) or from the grid; sKV: the workgroup's kv_lds_bytes<D>() of LDS.
template <int D, bool CAUSAL, bool WINDOW>
__device__ __forceinline__ void prefill_wg(const PrefillParams& p, const uint32_t bx,
                                           unsigned char* __restrict__ sKV) {
  constexpr int kBC = tile_keys<D>();   // keys per KV tile
  constexpr int kKT = kBC / 32;         // 32-key MFMA tiles per KV tile
  constexpr int KC = D / 16;          // 16-deep k-chunks of the QK^T contraction
  constexpr int DC = D / 32;          // 32-wide d chunks of O^T
  constexpr int ROWB = 2 * D;         // bytes per K/V row in LDS (unpadded, swizzled)
  constexpr int TPR = D / 8;          // lanes per row in a direct load (16 bytes each)
  constexpr int RPI = kWave / TPR;    // rows per direct-load instruction (4 or 8: divides 16)
  constexpr int NI = kBC / RPI;       // instructions per K (or V) tile
  // Every wave issues NI / 8 of a tile's direct loads (each a K and a V instruction), one after
  // every other k-chunk of its QK^T MFMAs: a wave stalls at issue while the CU's vector-memory
  // queue is full, so the loads of a whole tile issued in one burst held the issuing waves for
  // most of a thousand cycles per tile (s_memtime stamps on gfx950).
  constexpr int kDmaWaves = kWaves;
  constexpr int IPW = NI / kDmaWaves;   // of them issued by each wave
  constexpr int TILEB = kBC * ROWB;   // bytes of one K (or V) tile
  static_assert(IPW * kDmaWaves == NI, "tile rows must split evenly over the waves");

  // sKV: [buffer][K, V] tiles, row-major [key][d] with 16-byte chunks XOR-swizzled per row;
  // the next tile lands in one buffer while the other is consumed
  static_assert(kBufs * 2 * TILEB == kv_lds_bytes<D>(), "LDS size");

  const bool single = p.single_ql > 0;          // cascade prefix pass: one sequence
  const int group = p.num_heads / p.num_kv_heads;
  // The prologue's loads are issued side by side wherever their addresses allow (each
  // dependent scalar load would otherwise cost a full memory round trip before the first
  // K/V tile is requested): the schedule count and item together, then the request's
  // metadata together with the first tile's block ids.
  // kernel arguments, all requested before the first wait (an empty asm that reads them
  // keeps the compiler from loading each one behind its own branch)
  asm volatile("" ::"s"(p.q), "s"(p.kv), "s"(p.block_table), "s"(p.qsl), "s"(p.seq_lens),
               "s"(p.out), "s"(p.lse), "s"(p.v_offset), "s"(p.num_heads), "s"(p.num_kv_heads),
               "s"(p.block_size), "s"(p.max_blocks), "s"(p.seq_begin), "s"(p.window),
               "s"(p.scale), "s"(p.group_recip), "s"(p.kv_skip_blocks), "s"(p.single_ql),
               "s"(p.single_sl), "s"(p.single_slice), "s"(p.slice_stride), "s"(p.out_f32),
               "s"(p.schedule), "s"(p.max_qtiles), "s"(p.init_o), "s"(p.init_lse),
               "s"(p.num_seqs), "s"(gridDim.x));
  int r, qt, hq_grid;
  if (p.schedule != nullptr) {
    // item slot bx / num_heads of the schedule (sorted longest first), q head from
    // j = bx % num_heads; slots past the item count have nothing to do (the buffer holds an
    // entry for every slot, so the item load is in bounds). Workgroup ids go to the 8 XCDs
    // in turn and each XCD has its own L2, so when num_heads is a multiple of 8 the head is
    // (j % 8) * (num_heads / 8) + j / 8: the XCD of a workgroup then depends on its head
    // block only, and every q tile of a (request, kv head) - whose q heads share the K/V
    // tiles - runs on one XCD and reads them through one L2. (With the head = j order each
    // XCD read every kv head's K/V for every q tile: 6x the HBM/MALL fetches.)
    const int slot = bx / p.num_heads;
    const int count = p.schedule[0];
    const int e = p.schedule[1 + slot];
    asm volatile("" ::"s"(count), "s"(e));       // one wait for both loads
    if (slot >= count) return;
    r = p.seq_begin + e / p.max_qtiles;
    qt = e % p.max_qtiles;
    const int j = bx % p.num_heads;
    hq_grid = p.num_heads % 8 == 0 ? (j % 8) * (p.num_heads / 8) + j / 8 : j;
  } else {
    // the grid. Head size 128 with num_heads a multiple of 8 (not in the prefix pass): (q
    // tiles, heads, requests), read in its linear order, heads fastest, each request's
    // longest (causal) q tiles first. Otherwise (heads, requests, q tiles), q-tile-major: the
    // last q tile of every request (the heaviest under a causal mask; empty for short
    // requests, which return at once) before any earlier one. Head size 64 fits two
    // workgroups on a CU, and the q-tile-major order pairs heavy and light tiles on the CUs
    // where the request-major one paired equal ones (a 4 x 1024-token batch, 32 heads: 41.2
    // -> 32.5 us); for head size 128 (one workgroup per CU) the request-major order was 4 %
    // faster on the mixed workload's prefill rows. When num_heads is a multiple of 8 the
    // heads are placed on the XCDs as in the scheduled mode above. The prefix pass uses (q
    // tiles, kv heads, key slices). Written with selects rather than branches: with an if /
    // else-if / else here the compiler left the head undefined on one path (no copy of the
    // workgroup id y on that edge of the merged control flow).
    const bool remap = !single && p.num_heads % 8 == 0;
    const bool qmajor = !single && (D == 64 || p.num_heads % 8 != 0);
    const uint32_t id = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const uint32_t per_req = gridDim.x * (uint32_t)p.num_heads;
    const int local = (int)(id % per_req);
    const int j = qmajor ? (int)blockIdx.x : local % p.num_heads;
    r = single ? 0 : p.seq_begin + (qmajor ? (int)blockIdx.y : (int)(id / per_req));
    qt = single ? (int)gridDim.x - 1 - (int)blockIdx.x
                : (qmajor ? (int)gridDim.z - 1 - (int)blockIdx.z
                          : (int)gridDim.x - 1 - local / p.num_heads);
    hq_grid = single ? (int)blockIdx.y : (remap ? (j % 8) * (p.num_heads / 8) + j / 8 : j);
  }
  r = __builtin_amdgcn_readfirstlane(r);            // wave-uniform
  qt = __builtin_amdgcn_readfirstlane(qt);
  hq_grid = __builtin_amdgcn_readfirstlane(hq_grid);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave index, uniform
  const int lane = tid % kWave;
  const int dw = w % kDmaWaves;                     // direct-load slot of this wave
  const int32_t* __restrict__ bt = p.block_table + (int64_t)r * p.max_blocks + p.kv_skip_blocks;
  // Block ids of this wave's direct loads of tile 0, loaded beside the sequence metadata
  // (they depend on the request only), so that the first tile's loads wait for one memory
  // round trip less. They are used when the walk starts at tile 0 and tile 0 lies wholly
  // below seq_len (the ids are then those fetch_ids(0) would load). The index is clamped to
  // the block-table row and to the rows of this launch's requests, so the load is always in
  // bounds, and it is unconditional so that it is issued before the metadata is waited for.
  const int row_blocks = p.max_blocks - p.kv_skip_blocks;   // entries left in the row
  int32_t ids0, ids0_row_in_block;
  {
    const int u = min(lane, IPW - 1);
    const uint32_t grp = (uint32_t)(((dw + kDmaWaves * u) * RPI) >> 4);
    const int bi = min((int)(((uint64_t)grp * p.group_recip) >> 32), row_blocks - 1);
    const int64_t idx = min((int64_t)r * p.max_blocks + p.kv_skip_blocks + max(bi, 0),
                            (int64_t)(p.seq_begin + p.num_seqs) * p.max_blocks - 1);
    ids0 = p.block_table[idx];
    ids0_row_in_block = (int)grp * 16 - bi * p.block_size;
  }
  // The request's metadata (in the prefix pass r is 0, so these loads are valid there too):
  // three scalar loads and one wait for them, after the vector load above has been issued,
  // so the two round trips overlap. (The compiler would use vector loads here, since it
  // cannot prove that the kernel's stores leave this memory alone, and would wait for those
  // before issuing the block-id load.) Nothing writes this memory during the kernel.
  int qsl0, qsl1, slr;
  asm volatile(
      "s_load_dword %0, %3, 0x0\n\ts_load_dword %1, %3, 0x4\n\ts_load_dword %2, %4, 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(qsl0), "=&s"(qsl1), "=&s"(slr)   // early clobber: written before the inputs are read
      : "s"(p.qsl + r), "s"(p.seq_lens + r)
      : "memory");
  const int q_start = single ? 0 : qsl0;
  // query rows of this workgroup's sequence: its tokens, or in the prefix pass the
  // (token, q head) pairs of one GQA group
  const int ql = single ? p.single_ql * group : qsl1 - qsl0;
  // keys of this pass: [0, sl) after skipping kv_skip_blocks leading blocks
  const int sl = single ? p.single_sl : slr - p.kv_skip_blocks * p.block_size;
  if (qt * kBR >= ql) return;
  const int cl = sl - ql;
  const int kvh = single ? hq_grid : hq_grid / group;

  const int h = lane / 32;            // half-wave
  const int lq = lane % 32;           // query column of this lane

  const __bf16* __restrict__ q = static_cast<const __bf16*>(p.q);
  const __bf16* __restrict__ kcache = static_cast<const __bf16*>(p.kv);
  const __bf16* __restrict__ vcache = kcache + p.v_offset;

  // (token, q head) row of this lane's query column, as an index into [token][head] arrays
  const int wrow0 = qt * kBR + w * kRows;                // first query row of this wave
  const int my_row = min(wrow0 + lq, ql - 1);            // rows past ql: any valid row
  const int64_t my_th = single
      ? (int64_t)(my_row / group) * p.num_heads + kvh * group + my_row % group
      : (int64_t)(q_start + my_row) * p.num_heads + hq_grid;

  // ---- Q^T (B operand): lane l holds query lq, d = 16c + 8h .. +7
  bf16x8 qf[KC];
  {
    const __bf16* src = q + my_th * D + 8 * h;
#pragma unroll
    for (int c = 0; c < KC; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(src + 16 * c);
  }

  // ---- KV range of the workgroup and of this wave
  const int row_lo = qt * kBR;
  const int row_hi = min(ql, row_lo + kBR) - 1;
  const int kv_hi = CAUSAL ? min(sl, cl + row_hi + 1) : sl;
  const int kv_lo = WINDOW ? max(0, cl + row_lo - p.window + 1) : 0;
  int t_begin = kv_lo / kBC;
  int t_end = (kv_hi + kBC - 1) / kBC;
  if (single && p.single_slice > 0) {           // this workgroup's slice of the keys
    t_begin = (int)blockIdx.z * (p.single_slice / kBC);
    t_end = min(t_end, t_begin + p.single_slice / kBC);
  }
  const int w_row_lo = wrow0;
  const int w_row_hi = min(ql, wrow0 + kRows) - 1;
  const bool wave_active = w_row_lo <= w_row_hi;
  const int w_kv_hi = CAUSAL ? min(sl, cl + w_row_hi + 1) : sl;
  const int w_kv_lo = WINDOW ? max(0, cl + w_row_lo - p.window + 1) : 0;

  // ---- K/V tiles go from HBM straight into LDS (global_load_lds_dwordx4: lane l of one
  // instruction lands at LDS base + 16 l), so there is no register staging and no LDS store.
  // An instruction covers RPI consecutive rows; they lie in one 16-key group, which lies in
  // one cache block (block_size is a multiple of 16). The block ids of the groups of a tile's
  // instructions are loaded one tile ahead (lane u holds that of the wave's instruction u) and
  // turned into the cache row index of each group's first key (block * block_size + the
  // group's offset in its block); an instruction's address is then one multiply-add of that
  // row index (read back with v_readlane) with a per-lane base, which keeps the scalar unit
  // (shared by the CU's four SIMDs) nearly free of address arithmetic. Rows past seq_len load
  // row seq_len - 1: its scores are masked and 0 * (finite V) adds nothing, so no zeroing is
  // needed. Because the destination of a lane is fixed, the row layout is permuted on the
  // source side: LDS chunk slot p of row r holds d-chunk p ^ swz(r), which keeps both MFMA
  // operand reads free of bank conflicts.
  const int kv_row = p.num_kv_heads * D;
  const uint32_t row_bytes = (uint32_t)(kv_row * 2);
  const int last_group = (sl - 1) >> 4;
  const int l_row = lane / TPR;                      // row of this lane within an instruction
  const int l_slot = lane % TPR;                     // LDS chunk slot of this lane
  // group index of the first row of direct-load instruction u (u < IPW) of this wave in a tile
  auto group_of = [&](int tile, int u) {
    return min((tile * kBC + (dw + kDmaWaves * u) * RPI) >> 4, last_group);
  };
  auto block_index = [&](int grp) {
    return (uint32_t)(((uint64_t)(uint32_t)grp * p.group_recip) >> 32);
  };
  // Groups of a tile's IPW instructions (lane u < IPW: instruction u; group_of clamps to the
  // last group, so every index is a valid entry of the request's row): fetch_ids loads their
  // block ids and keeps each group's offset in its block; row_base, once the load has landed,
  // gives the cache row index of each group's first key.
  struct Ids {
    int32_t blk;
    int32_t row_in_block;
  };
  auto fetch_ids = [&](int tile) {
    const int grp = group_of(tile, min(lane, IPW - 1));
    const uint32_t bidx = block_index(grp);
    return Ids{bt[bidx], grp * 16 - (int)bidx * p.block_size};
  };
  auto row_base = [&](const Ids& ids) {
    return (uint32_t)ids.blk * (uint32_t)p.block_size + (uint32_t)ids.row_in_block;
  };
  // Per-lane byte part of the source addresses: kv head and d-chunk l_slot ^ swizzle(row) (the
  // swizzle depends on the row modulo 16 only, which is the same for every instruction of this
  // wave: j RPI = dw RPI mod 16).
  const uint32_t chunk_bytes =
      (uint32_t)(kvh * D * 2 + 16 * (l_slot ^ swizzle<D>(dw * RPI + l_row)));
  const unsigned char* const k_lane = reinterpret_cast<const unsigned char*>(kcache) + chunk_bytes;
  const unsigned char* const v_lane = reinterpret_cast<const unsigned char*>(vcache) + chunk_bytes;
  // the K and V direct loads of this wave's instruction u of a tile into buffer buf; rb holds
  // the row bases of the tile's groups. The lane's key is clamped to seq_len - 1 (a no-op for
  // tiles wholly below seq_len), so the same arithmetic serves full and tail tiles.
  auto issue_one = [&](int tile, int buf, uint32_t rb, int u) {
    const int j = dw + kDmaWaves * u;                // instruction index within the tile
    const uint32_t rbu = __builtin_amdgcn_readlane(rb, u);
    const int key = min(tile * kBC + j * RPI + l_row, sl - 1);
    const uint32_t row = rbu + (uint32_t)(key - group_of(tile, u) * 16);
    const uint32_t lds_k = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(sKV + buf * (2 * TILEB) + j * (RPI * ROWB)));
    dma_b128(k_lane + (uint64_t)row * row_bytes, lds_k);
    dma_b128(v_lane + (uint64_t)row * row_bytes, lds_k + TILEB);
  };
  auto issue_tile = [&](int tile_in, int buf, uint32_t rb) {
    // the tile index is wave-uniform; saying so keeps its arithmetic scalar
    const int tile = __builtin_amdgcn_readfirstlane(tile_in);
#pragma unroll
    for (int u = 0; u < IPW; ++u) issue_one(tile, buf, rb, u);
  };

  // per-lane byte offsets of the transposing V reads within a tile for (kt, g) = (0, 0):
  // logical column 32dc + 16((lane/16)%2) + 4(lane%4) is 16-byte chunk
  // 4dc + 2((lane/16)%2) + (lane%4)/2, plus 8 bytes when lane%4 is odd
  uint32_t v_off0[DC], v_off1[DC];
  {
    const int rr = 4 * h + (lane % 16) / 4;
    const int cchunk = 2 * ((lane / 16) % 2) + (lane % 4) / 2;
    const int cbyte = 8 * (lane % 2);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const int ch = 4 * dc + cchunk;
      v_off0[dc] = rr * ROWB + 16 * (ch ^ swizzle<D>(rr)) + cbyte;
      v_off1[dc] = (rr + 8) * ROWB + 16 * (ch ^ swizzle<D>(rr + 8)) + cbyte;
    }
  }

  const float c_log2 = p.scale * kLog2e;
  float m_ref = -INFINITY;
  float l_run = 0.f;        // per-lane partial row sum (fp32: the lse needs it unrounded)
  floatx16 o[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dc][e] = 0.f;

  // A partial result over earlier keys (out o0 normalised, log-sum-exp lse0) is the state
  // O = o0, l = 1 with the reference max m = lse0 / scale: the prefix's sum of
  // exp(scale (s - m)) is exp(lse0 - scale m) = 1.
  if (p.init_o != nullptr) {
    const int64_t ri = my_th;
    const float lse0 = p.init_lse[ri];
    if (lse0 > -INFINITY) {
      m_ref = lse0 / p.scale;
      l_run = h == 0 ? 1.f : 0.f;                // the lane pair's partial sums add up to 1
      const float* src = p.init_o + ri * D + 4 * h;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const floatx4 v = *reinterpret_cast<const floatx4*>(src + 32 * dc + 8 * e4);
#pragma unroll
          for (int i = 0; i < 4; ++i) o[dc][4 * e4 + i] = v[i];
        }
    }
  }

  Ids ids{0, 0};
  if (t_begin < t_end) {
    Ids first_ids;
    if (t_begin == 0 && kBC <= sl && row_blocks > 0) first_ids = Ids{ids0, ids0_row_in_block};
    else first_ids = fetch_ids(t_begin);
    issue_tile(t_begin, 0, row_base(first_ids));
    ids = fetch_ids(t_begin + 1);      // clamped to the last group: always a valid entry
  }
  wait_vmem();                         // Q, tile t_begin and the ids of tile t_begin + 1
  barrier_kv();
  int buf = 0;
  for (int t = t_begin; t < t_end; ++t) {
    // tile t + 1 goes to the other buffer, which every wave finished reading (tile t - 1)
    // before the barrier that ended the previous iteration. Its loads are issued whether or
    // not a tile t + 1 exists (past the last tile they reload the last rows into a buffer no
    // one reads again), which keeps them free of branches between the QK^T MFMAs.
    const uint32_t rb_next = row_base(ids);
    const int t_next = __builtin_amdgcn_readfirstlane(t + 1);
    ids = fetch_ids(t + 2);

    const int kb = t * kBC;
    if (wave_active && kb < w_kv_hi && kb + kBC > w_kv_lo) {
      const unsigned char* tK = sKV + buf * (2 * TILEB);
      const unsigned char* tV = tK + TILEB;
      // S^T: sc[kt] element e holds key kb + 32kt + 8(e/4) + 4h + e%4 of query column lq
      floatx16 sc[kKT];
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[kt][e] = 0.f;
      {
        // K row kt*32 + lq has the swizzle of row lq (it depends on the row modulo 16)
        const int ks = swizzle<D>(lq);
        const unsigned char* kp = tK + lq * ROWB;
        constexpr int kGap = KC / IPW;               // chunks between this wave's loads
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const int off = 16 * ((2 * c + h) ^ ks);
#pragma unroll
          for (int kt = 0; kt < kKT; ++kt)
            sc[kt] = mfma32x32x16(
                *reinterpret_cast<const bf16x8*>(kp + kt * 32 * ROWB + off), qf[c], sc[kt]);
          if (c % kGap == 0) issue_one(t_next, buf ^ 1, rb_next, c / kGap);
        }
        // software pipeline: the K operands of chunk c + 1 are read while chunk c multiplies
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kKT, 0);   // LDS reads
#pragma unroll
        for (int c = 0; c + 1 < KC; ++c) {
          __builtin_amdgcn_sched_group_barrier(0x008, kKT, 0);     // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, kKT, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kKT, 0);
      }

      const bool need_mask = (kb + kBC > sl) || (CAUSAL && kb + kBC - 1 > cl + w_row_lo) ||
                             (WINDOW && kb < cl + w_row_hi - p.window + 1);
      if (need_mask) {
        const int pos = cl + wrow0 + lq;             // absolute position of this query
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int j = kb + 32 * kt + 8 * (e / 4) + 4 * h + (e % 4);
            bool vis = j < sl;
            if (CAUSAL) vis = vis && (j <= pos);
            if (WINDOW) vis = vis && (j >= pos - p.window + 1);
            if (!vis) sc[kt][e] = -INFINITY;
          }
      }

      // online softmax with a lazily moved reference max, one query column per lane pair;
      // the row max and row sum use 8 independent partial results (short dependency
      // chains) combined by a tree
      // (each chain starts from three scores and takes two more per three-input maximum)
      float pm[8];
      {
        constexpr int NS = 16 * kKT;                 // scores per lane
#define SC(n) sc[(n) / 16][(n) % 16]
#pragma unroll
        for (int i = 0; i < 8; ++i) pm[i] = max3_f32(SC(3 * i), SC(3 * i + 1), SC(3 * i + 2));
#pragma unroll
        for (int n = 24; n + 1 < NS; n += 2) {
          const int i = ((n - 24) / 2) % 8;
          pm[i] = max3_f32(pm[i], SC(n), SC(n + 1));
        }
        if constexpr (NS % 2 == 1) pm[0] = max_f32(pm[0], SC(NS - 1));
#undef SC
      }
      float mx = max3_f32(max3_f32(pm[0], pm[1], pm[2]), max3_f32(pm[3], pm[4], pm[5]),
                          max_f32(pm[6], pm[7]));
      {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                  false, false);
        mx = max_f32(__uint_as_float(r[0]), __uint_as_float(r[1]));
      }
      // move the reference when the tile max exceeds it by more than 2^kRescaleLog2
      // (always on a column's first visible key, where m_ref is -inf)
      const bool move = (mx - m_ref) * c_log2 > kRescaleLog2;
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
        // alpha is 0 when m_ref was -inf; columns that keep their reference use 1
        const float alpha = move ? fast_exp2((m_ref - mx) * c_log2) : 1.f;
        if (move) m_ref = mx;
        l_run *= alpha;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) o[dc] *= alpha;
      }
      const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * c_log2;
      float ps[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ps[i] = 0.f;
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          sc[kt][e] = fast_exp2(fmaf(sc[kt][e], c_log2, -mc));
          ps[e % 8] += sc[kt][e];
        }
      l_run += ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]));

      // O^T += V^T . P^T, one MFMA per 16 keys: MFMA (kt, g) contracts keys
      // kb + 32kt + 16g + 8(j/4) + 4h + j%4 at k = 8h + j. P^T is elements 8g .. 8g+7 of
      // sc[kt]; V^T comes from two transposing reads of 4 rows each (rows r0 and r0 + 8,
      // r0 = 32kt + 16g + 4h + (lane%16)/4), whose addresses differ from the (kt, g) = (0, 0)
      // ones by a constant because the swizzle depends on the row modulo 16 only.
      const uint32_t tv_addr = (uint32_t)(uintptr_t)tV;
      uint32_t va0[DC], va1[DC];
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        va0[dc] = tv_addr + v_off0[dc];
        va1[dc] = tv_addr + v_off1[dc];
      }
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const floatx4 lo = {sc[kt][8 * g + 0], sc[kt][8 * g + 1], sc[kt][8 * g + 2],
                              sc[kt][8 * g + 3]};
          const floatx4 hi = {sc[kt][8 * g + 4], sc[kt][8 * g + 5], sc[kt][8 * g + 6],
                              sc[kt][8 * g + 7]};
          const bf16x8 pb = pack_bf16x8(lo, hi);
          const uint32_t step = (32 * kt + 16 * g) * ROWB;
#pragma unroll
          for (int dc = 0; dc < DC; ++dc) {
            const bf16x8 va = concat(tr_read(lds_at(va0[dc] + step)),
                                     tr_read(lds_at(va1[dc] + step)));
            o[dc] = mfma32x32x16(va, pb, o[dc]);
          }
        }
      {
        // software pipeline: the V^T operands of the next L MFMAs are read while one
        // multiplies (left to itself the scheduler read them one MFMA ahead for d = 128 and
        // not at all for d = 64; L = 1 keeps d = 64 within the 128 registers of two
        // workgroups per CU; measured: the d = 64 workloads 2-3 % faster, d = 128 level to
        // 1 % faster)
        constexpr int L = D == 64 ? 1 : 2;
        constexpr int NM = kKT * 2 * DC;             // PV MFMAs per tile
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * L, 0);   // LDS reads
#pragma unroll
        for (int m = 0; m + L < NM; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, L, 0);
      }
    } else {
      issue_tile(t_next, buf ^ 1, rb_next);         // a wave with nothing to compute here
    }
    wait_vmem();        // this wave's part of tile t + 1 is in LDS ...
    barrier_kv();       // ... and everyone's, and nobody reads tile t any more
    buf ^= 1;
  }

  // ---- epilogue: O / l and lse = scale * m + ln l
  const float l_tot = add_xor32(l_run);
  const int row = wrow0 + lq;
  if (row < ql) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t th = my_th + (single ? (int64_t)blockIdx.z * p.slice_stride : 0);
    const int64_t off = th * D + 4 * h;
    if (p.out_f32 != nullptr) {
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
          *reinterpret_cast<floatx4*>(p.out_f32 + off + 32 * dc + 8 * e4) =
              floatx4{o[dc][4 * e4 + 0] * inv, o[dc][4 * e4 + 1] * inv,
                      o[dc][4 * e4 + 2] * inv, o[dc][4 * e4 + 3] * inv};
    } else {
      // A lane holds d = 32 dc + 8 e4 + 4h .. +3 of its row for every 8-wide chunk e4. The two
      // lanes of a row (l and l ^ 32, always both active) trade halves so that each ends with
      // 8 consecutive d of one chunk (e4 = 2 pe + h) and writes them as one 16-byte store,
      // half the store instructions of writing 4-element runs.
      __bf16* dst = static_cast<__bf16*>(p.out) + th * D;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int pe = 0; pe < 2; ++pe) {
          floatx4 lo, hi;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a = o[dc][4 * (2 * pe) + i] * inv;        // chunk 2 pe, this lane's half
            const float b = o[dc][4 * (2 * pe + 1) + i] * inv;    // chunk 2 pe + 1
            const float got = __shfl_xor(h ? a : b, 32);
            lo[i] = h ? got : a;
            hi[i] = h ? b : got;
          }
          *reinterpret_cast<bf16x8*>(dst + 32 * dc + 8 * (2 * pe + h)) = pack_bf16x8(lo, hi);
        }
    }
    if (p.lse != nullptr && h == 0) {
      p.lse[th] =
          l_tot > 0.f ? p.scale * m_ref + __logf(l_tot) : -INFINITY;
    }
  }
}

template <int D, bool CAUSAL, bool WINDOW>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(const PrefillParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char sKV[kv_lds_bytes<D>()];
  prefill_wg<D, CAUSAL, WINDOW>(p, blockIdx.x, sKV);
}

// One launch for one layer pass of a mixed batch: the first dec_wgs workgroups take the decode
// rows, each wave a (decode request, kv head, head group) unit at a time streaming the
// request's visible keys and writing its output (dec::decode_request_wave: no partitions, no
// merge, no workspace), so the HBM-bound decode waves start at once on dec_wgs CUs; the other
// workgroups are the prefill kernel's scheduled slots (p.schedule, sorted longest first).
// Both kinds share one LDS allocation (the larger of their needs).
constexpr int kMixedDecodeWgs = 64;
template <int D, bool CAUSAL, bool WINDOW>
__global__ __launch_bounds__(kThreads, 2) void mixed_bf16_kernel(const PrefillParams p,
                                                                 const DecodeParams dp,
                                                                 const int32_t dec_wgs) {
  using T = dec::WaveTiles<D>;
  constexpr int kWaveLds = (T::V_TILE + T::K_TILE) * 2;     // bytes of one decode wave's tiles
  constexpr int kLds = kv_lds_bytes<D>() > kWaves * kWaveLds ? kv_lds_bytes<D>()
                                                               : kWaves * kWaveLds;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kLds];
  if ((int)blockIdx.x < dec_wgs) {
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int heads_wg = dp.num_kv_heads * ((dp.num_heads / dp.num_kv_heads + 15) / 16);
    __bf16* tiles = reinterpret_cast<__bf16*>(lds + w * kWaveLds);
    if (heads_wg % 8 == 0 && dec_wgs % 8 == 0) {
      // Workgroup b runs on XCD b % 8 (each XCD has its own L2): its waves take only the
      // (kv head, head group) units hw with hw % 8 == b % 8, every request in turn, so each
      // XCD streams one eighth of the heads (the prefill workgroups of those kv heads' q heads
      // run on the same XCD) and the shared prefix of a head is read by the waves of one L2.
      const int x = (int)blockIdx.x % 8;
      const int hpx = heads_wg / 8;                  // units per request on this XCD
      const int n = dp.num_decodes * hpx;
      for (int i = ((int)blockIdx.x / 8) * kWaves + w; i < n; i += (dec_wgs / 8) * kWaves)
        dec::decode_request_wave<D>(dp, i / hpx, x + 8 * (i % hpx), tiles, tiles + T::V_TILE);
      return;
    }
    for (int unit = (int)blockIdx.x * kWaves + w; unit < dp.num_decodes * heads_wg;
         unit += dec_wgs * kWaves)
      dec::decode_request_wave<D>(dp, unit / heads_wg, unit % heads_wg, tiles,
                                  tiles + T::V_TILE);
    return;
  }
  prefill_wg<D, CAUSAL, WINDOW>(p, blockIdx.x - (uint32_t)dec_wgs, lds);
}

template <int D, bool CAUSAL, bool WINDOW>
hipError_t launch_mixed(const PrefillParams& p, const DecodeParams& dp, hipStream_t stream) {
  const int heads_wg = dp.num_kv_heads * ((dp.num_heads / dp.num_kv_heads + 15) / 16);
  // decode workgroups: one wave per unit up to kMixedDecodeWgs workgroups (their waves then
  // take several units each) - enough waves to keep HBM busy while the CUs they hold are
  // taken from the prefill work
  const int64_t dec_wgs = std::min<int64_t>(
      ((int64_t)dp.num_decodes * heads_wg + kWaves - 1) / kWaves, kMixedDecodeWgs);
  const int64_t pre_wgs = p.num_seqs > 0 ? (int64_t)p.num_seqs * p.max_qtiles * p.num_heads : 0;
  if (dec_wgs + pre_wgs == 0) return hipSuccess;
  hipLaunchKernelGGL((mixed_bf16_kernel<D, CAUSAL, WINDOW>), dim3((unsigned)(dec_wgs + pre_wgs)),
                     dim3(kThreads), 0, stream, p, dp, (int32_t)dec_wgs);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool WINDOW>
hipError_t launch(const PrefillParams& p, hipStream_t stream) {
  const unsigned qtiles = (unsigned)((p.max_query_len + kBR - 1) / kBR);
  // (q tiles, heads, requests), request-major, or (heads, requests, q tiles), q-tile-major
  // (the orders are explained in prefill_wg)
  dim3 grid = D == 128 && p.num_heads % 8 == 0 ? dim3(qtiles, p.num_heads, p.num_seqs)
                                               : dim3(p.num_heads, p.num_seqs, qtiles);
  if (p.schedule != nullptr) {       // one workgroup per (schedule slot, q head)
    grid = dim3((unsigned)((int64_t)p.num_seqs * p.max_qtiles * p.num_heads), 1, 1);
  } else if (p.single_ql > 0) {            // prefix pass: (token, head) rows per kv head, key slices
    const int rows = p.single_ql * (p.num_heads / p.num_kv_heads);
    const int slices = p.single_slice > 0 ? (p.single_sl + p.single_slice - 1) / p.single_slice : 1;
    grid = dim3((rows + kBR - 1) / kBR, p.num_kv_heads, slices);
  }
  hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, WINDOW>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mask(const PrefillParams& p, hipStream_t stream) {
  if (p.window > 0) return launch<D, true, true>(p, stream);
  if (p.causal) return launch<D, true, false>(p, stream);
  return launch<D, false, false>(p, stream);
}

template <int D>
hipError_t launch_mixed_mask(const PrefillParams& p, const DecodeParams& dp,
                             hipStream_t stream) {
  if (p.window > 0) return launch_mixed<D, true, true>(p, dp, stream);
  if (p.causal) return launch_mixed<D, true, false>(p, dp, stream);
  return launch_mixed<D, false, false>(p, dp, stream);
}

}  // namespace

hipError_t launch_mixed_bf16(const PrefillParams& p, const DecodeParams& dp,
                             hipStream_t stream) {
  return p.head_size == 64 ? launch_mixed_mask<64>(p, dp, stream)
                           : launch_mixed_mask<128>(p, dp, stream);
}

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream) {
  if (p.num_seqs <= 0 || p.max_query_len <= 0) return hipSuccess;
  return p.head_size == 64 ? launch_mask<64>(p, stream) : launch_mask<128>(p, stream);
}

}  // namespace attn
