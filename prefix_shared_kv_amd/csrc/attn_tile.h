#pragma once
// Shared attention tile for extend and decode (included by extend.hip and
// decode.hip): attention over a prefix-shared KV pool, gfx950.
//
// What is computed follows the "Prompt Caching" glossary, section "How prompt
// caching works" and its GPT-2 example: a request's new tokens attend causally,
// by absolute position, over the cached K/V of its prefix and over their own
// K/V; a decode token attends over the whole context.  The result equals a full
// recompute up to floating-point rounding (the page's closing "related terms").
//
// One MFMA kernel serves both.  A workgroup of NW waves (4 for decode, 8 for
// extend) owns up to 32 NW query "columns" that read the same kv head over
// the same key positions:
//   extend : columns = (new token, q head of the kv head's group) of one request
//   decode : columns = (member request, q head) of one plan item, i.e. every
//            request whose context holds this range of slots — a prefix shared
//            by many branches is loaded from HBM once for all of them.
// Keys are processed in stages of 64.  Each stage is gathered from the pool
// through the request->slot table (or read from k_new/v_new for the extend's
// own tokens), staged in LDS — K row-major, V transposed — and consumed by
//   S^T = K Q^T    (v_mfma_f32_32x32x16_bf16, rows = keys, columns = queries)
//   O^T += V^T P^T (same instruction, rows = head dims)
// Computing S transposed puts one query column per lane: the softmax max and
// the rescale of O are in-lane, plus one exchange between lanes l and l^32
// per stage.  The 16 keys a lane holds for one PV step come straight from the
// S^T accumulator; V^T is stored in LDS with the matching key permutation so
// each MFMA operand is one 16-byte LDS read.  Online softmax runs in base 2
// with log2(e) folded into the scale.
#include <cfloat>
#include <cmath>
#include <type_traits>

#include "hip_common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BN = 64;     // keys per stage
constexpr int NT = 256;
constexpr float LOG2E = 1.4426950408889634f;

enum Mode { EXTEND = 0, DECODE = 1 };

struct Args {
  const void* q;
  void* o;
  const void* k_new;
  const void* v_new;
  const void* k_pool;
  const void* v_pool;
  const int32_t* table;
  int32_t table_rows;
  int64_t stride;      // table entries per row
  int64_t pool_slots;
  int32_t page_shift;  // log2(page size): table entries are page ids when > 0
  int32_t Hq, Hkv, g;
  float scale_log2;  // sm_scale * log2(e)
  int32_t* err;
  int32_t n_work;    // workgroups in the grid
  // extend
  const int32_t* rows;
  const int32_t* prefix_lens;
  const int32_t* extend_lens;
  const int32_t* extend_start;
  int32_t batch;
  int32_t max_extend;
  int64_t total_extend;
  int32_t tiles;     // tiles per (request, kv head)
  int32_t tok_per_tile;
  // decode
  const int32_t* plan;
  const int32_t* new_slots;    // decode: pool slot of each request's current token (with k_new/v_new)
  int32_t n_items, n_members;  // from the planner's host summary
  int32_t narrow_begin;        // first item with members*group <= 16
  int32_t narrow_first;        // workgroups run the narrow items first, then the wide ones
  int32_t n_wide_blocks;       // workgroups that run wide items
  int32_t n_narrow_units;      // (narrow item, kv head) pairs, one wave each
  int32_t max_cols;            // query columns of the launch's tile (32 per wave)
  const int32_t* seq_lens;
  void* ws_o;    // partial outputs: bf16 rows for bf16 data, fp32 rows for fp32
  float* ws_ml;
  int32_t max_splits;
};

// What one workgroup computes, resolved from the grid position.
struct Work {
  bool valid;
  int32_t hk;
  int64_t row;         // table row for positions < ext_begin
  int32_t key_begin, key_end;
  int32_t ext_begin;   // positions >= ext_begin come from k_new/v_new
  int64_t ext_base;    // token index in k_new of position ext_begin
  int32_t ncols;
  int32_t min_limit;   // smallest causal limit over the columns
  // extend
  int32_t t0, E, P;
  // decode
  int32_t split, moff, mcnt;
  int32_t store_b;     // request whose current token this item stores and reads from k_new (-1: none)
};

__device__ __forceinline__ void flag(int32_t* err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

// Position p's slot from its table entry: one entry per position, or with
// paging (shift > 0) one page id per 2^shift positions, a page's slots being
// consecutive.  A page id outside the pool gives -1, an invalid slot.
__device__ __forceinline__ int32_t page_slot(int32_t entry, int p, int shift, uint32_t n_pages) {
  return (uint32_t)entry < n_pages ? (entry << shift) | (p & ((1 << shift) - 1)) : -1;
}

__device__ Work resolve(const Args& a, int mode, int L, bool leader) {
  Work w{};
  w.valid = false;
  w.store_b = -1;
  if (mode == EXTEND) {
    const int tile = L % a.tiles;
    const int bh = L / a.tiles;
    const int b = bh / a.Hkv;
    w.hk = bh - b * a.Hkv;
    const int P = a.prefix_lens[b], E = a.extend_lens[b];
    if (P < 0 || E < 0) {
      if (tile == 0 && leader) flag(a.err, RC_DEVERR_LENGTH);
      return w;
    }
    if (E > a.max_extend && tile == 0 && w.hk == 0 && leader) flag(a.err, RC_DEVERR_LENGTH);
    if ((int64_t)P > (a.stride << a.page_shift) || (P > 0 && a.pool_slots < 1)) {
      if (tile == 0 && leader) flag(a.err, RC_DEVERR_TABLE);
      return w;
    }
    const int t0 = tile * a.tok_per_tile;
    const int Ec = E < a.max_extend ? E : a.max_extend;
    if (t0 >= Ec) return w;
    const int nt = min(a.tok_per_tile, Ec - t0);
    const int64_t s0 = a.extend_start[b];
    if (s0 < 0 || s0 + Ec > a.total_extend) {
      if (tile == 0 && leader) flag(a.err, RC_DEVERR_LENGTH);
      return w;
    }
    w.row = a.rows ? a.rows[b] : b;
    if (w.row < 0 || w.row >= a.table_rows) {
      if (leader) flag(a.err, RC_DEVERR_TABLE);
      return w;
    }
    w.key_begin = 0;
    w.key_end = P + t0 + nt;
    w.ext_begin = P;
    w.ext_base = s0;
    w.ncols = nt * a.g;
    w.min_limit = P + t0;
    w.t0 = t0;
    w.E = Ec;
    w.P = P;
    w.valid = true;
  } else {
    const int item = L / a.Hkv;
    w.hk = L - item * a.Hkv;
    const int32_t* it = a.plan + RC_PLAN_HEADER + (int64_t)item * RC_PLAN_ITEM;
    const int32_t n_members = a.n_members;
    const int32_t rep = it[0], pb = it[1], pe = it[2];
    w.split = it[3];
    w.moff = it[4];
    w.mcnt = it[5];
    if (rep < 0 || rep >= a.table_rows || pb < 0 || pe < pb || (int64_t)pe > (a.stride << a.page_shift) ||
        a.pool_slots < 1 ||
        w.split < 0 || w.split >= a.max_splits ||
        w.moff < 0 || w.mcnt < 1 || w.mcnt * a.g > a.max_cols || w.moff + w.mcnt > n_members) {
      if (leader) flag(a.err, RC_DEVERR_PLAN);
      return w;
    }
    const int32_t* mem = a.plan + RC_PLAN_HEADER + (int64_t)a.n_items * RC_PLAN_ITEM + w.moff;
    for (int i = 0; i < w.mcnt; ++i)
      if (mem[i] < 0 || mem[i] >= a.batch) {
        if (leader) flag(a.err, RC_DEVERR_PLAN);
        return w;
      }
    const int sl = a.seq_lens[mem[0]];
    w.row = rep;
    w.key_begin = pb;
    w.key_end = pe < sl ? pe : sl;
    if (w.key_end < w.key_begin) w.key_end = w.key_begin;
    w.ext_begin = INT_MAX;
    w.ext_base = 0;
    w.store_b = -1;
    // The piece of a request's own range (marked by the planner) holding its
    // last position takes the current token's K/V from k_new/v_new and writes
    // them to the pool; a shared range is never written.
    if (a.k_new && (it[6] & RC_PLAN_ITEM_OWN) && w.mcnt == 1 && sl >= 1 && pb <= sl - 1 && pe >= sl) {
      w.ext_begin = sl - 1;
      w.ext_base = mem[0];
      w.store_b = mem[0];
    }
    w.ncols = w.mcnt * a.g;
    w.min_limit = INT_MAX;
    w.valid = true;
  }
  return w;
}

// Copy request b's current-token K and V row of kv head hk into its pool slot
// (threads [0, n) of the caller, 8 elements each; n = D / 8 covers the row).
template <typename T, int D>
__device__ __forceinline__ void store_new_token(const Args& a, int b, int hk, int t) {
  constexpr int VEC = 16 / sizeof(T);
  if (t >= D / VEC) return;
  const int32_t s = a.new_slots[b];
  if ((uint32_t)s >= (uint32_t)a.pool_slots) {
    if (t == 0) flag(a.err, RC_DEVERR_SLOT);
    return;
  }
  const int64_t src = ((int64_t)b * a.Hkv + hk) * D + t * VEC;
  const int64_t dst = ((int64_t)s * a.Hkv + hk) * D + t * VEC;
  *(uint4*)((T*)a.k_pool + dst) = *(const uint4*)((const T*)a.k_new + src);
  *(uint4*)((T*)a.v_pool + dst) = *(const uint4*)((const T*)a.v_new + src);
}

// Per-column (query) information.
struct Col {
  int64_t qoff;   // element offset of the query row (token, head)
  int32_t limit;  // last visible key position
  int32_t head;
  int32_t b;      // decode: batch index
  bool real;
};

__device__ __forceinline__ Col column(const Args& a, int mode, const Work& w, int c) {
  Col k;
  k.real = c < w.ncols;
  const int cc = k.real ? c : w.ncols - 1;
  const int u = cc / a.g, j = cc - (cc / a.g) * a.g;
  k.head = w.hk * a.g + j;
  if (mode == EXTEND) {
    const int t = w.t0 + u;
    k.qoff = (w.ext_base + t) * (int64_t)a.Hq + k.head;
    k.limit = w.P + t;
    k.b = -1;
  } else {
    const int32_t* mem = a.plan + RC_PLAN_HEADER + (int64_t)a.n_items * RC_PLAN_ITEM + w.moff;
    k.b = mem[u];
    k.qoff = (int64_t)k.b * a.Hq + k.head;
    k.limit = INT_MAX;
  }
  return k;
}

// LDS tiles hold K and V row-major, [key][head dim], with the 16-byte chunks
// of each row XOR-swizzled by a function of the key.  For D = 128 (256-byte
// rows, so the row itself never moves a bank) the swizzle is a linear
// bijection of the key's low 4 bits, found by exhaustive search over a model
// of 64 four-byte banks, that leaves every read pattern here free of bank
// conflicts: 16 keys reading one chunk (K operands, ds_read_b128, 16 lanes
// per pass), and the transposing V reads (32 lanes per pass) of both tile
// shapes: 4 keys x 4 chunks (32x32x16) and 8 keys x 2 chunks (16x16x32).
template <int D>
__device__ __forceinline__ int swz(int key) {
  if constexpr (D == 128)
    return ((key & 3) << 2) | ((key >> 1) & 2) | ((key >> 3) & 1);
  else
    return key & 7;
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return (lo16 & 0xffffu) | (hi16 << 16); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// Transposing LDS read (gfx950): within each 16-lane group, lane j receives
// element j%4 of the 8-byte blocks addressed by lanes j/4, 4+j/4, 8+j/4 and
// 12+j/4.  Lanes addressing 4 keys x 4 column blocks therefore receive a
// 16 (head dims) x 4 (keys) tile: one lane per head dim, 4 keys each.
__device__ __forceinline__ i16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// Lazy rescaling: a column's reference maximum moves only when a score
// exceeds it by more than this many powers of two, so p = 2^(s - m) stays
// below 2^8 and the O accumulator is rescaled a few times per tile instead of
// whenever the running maximum creeps up.  Partials and the final o = acc / l
// are exact up to rounding for any reference maximum.
constexpr float RESCALE_SLACK = 8.f;

// STREAM: K/V loads are nontemporal (decode steps read each range once per
// launch; extends re-read a prefix across tiles and keep it in L2).
//
// Keys whose table entry gives no valid pool slot are absent from the
// softmax.  The usual pass loads such a key from a clamped slot (every load
// stays inside the pool) and only notes it; if any lane of the workgroup met
// one, it writes nothing and returns true, and the caller runs the item again
// with CAREFUL set: that pass loads zeros for those keys and gives them a -inf
// score by reading each key's table entry beside its score.  The check costs
// the usual pass one workgroup-wide OR per item.
template <int D, int NW = 4, bool STREAM = false, bool CAREFUL = false>
__device__ __forceinline__ bool attn_bf16_body(const Args& a, const int mode, const int L, uint16_t (&sK)[2][BN * D],
                                               uint16_t (&sV)[2][BN * D]) {
  constexpr int CH = D / 8;                 // 16-byte chunks per key row
  constexpr int KPT = BN * CH / (64 * NW);  // keys per thread per stage
  constexpr int NKS = D / 16;        // MFMA k-steps over D
  constexpr int NDB = D / 32;        // 32-row blocks of O^T
  const Work w = resolve(a, mode, L, threadIdx.x == 0);
  if (!w.valid) return false;  // uniform over the workgroup
  // set by lanes that met an invalid slot; cleared before the first stage
  // barrier, so no lane can set it earlier
  __shared__ int32_t s_absent;
  if (!CAREFUL && threadIdx.x == 0) s_absent = 0;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS block addresses stay scalar
  const int hi = lane >> 5;  // which half of the wave
  const int c = wave * 32 + (lane & 31);
  const bool active = wave * 32 < w.ncols;
  const Col col = column(a, mode, w, c);
  if (w.store_b >= 0) store_new_token<uint16_t, D>(a, w.store_b, w.hk, tid);

  const uint16_t* q = (const uint16_t*)a.q;
  bf16x8 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8*)(q + col.qoff * D + ks * 16 + 8 * hi);

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // Loader.  Global -> LDS loads (global_load_lds_dwordx4) move 16 bytes per
  // lane into 1 KiB of LDS at lane-consecutive addresses, so each load
  // instruction fills one block of KPB keys x CH chunks of the row-major,
  // chunk-swizzled tile; a lane fetches the logical chunk that belongs at its
  // position.  Load r of wave w fills block NW r + w of K and of V: a lane's
  // keys are then NW*KPB apart, the same in the swizzle, so one column offset
  // serves all of them.
  constexpr int KPB = 64 / CH;  // keys per 1 KiB block
  const uint32_t row_bytes = (uint32_t)(a.Hkv * D * 2);
  const uint32_t nslots = (uint32_t)a.pool_slots;  // >= 1 (checked when the work is resolved)
  const int plain_end = min(w.key_end, w.ext_begin);  // stages ending here read pool slots only
  const int lkey0 = wave * KPB + lane / CH;           // this lane's key in block w; + r*4*KPB in block 4r+w
  const int coff = (w.hk * D + (((lane % CH) ^ swz<D>(lkey0)) << 3)) * 2;
  // this lane's chunk in slot 0 / new token 0; + index x row_bytes
  const char* kcol = (const char*)a.k_pool + coff;
  const char* vcol = (const char*)a.v_pool + coff;
  const char* kncol = (const char*)a.k_new + coff;
  const char* vncol = (const char*)a.v_new + coff;
  // k_new / v_new relative to the pools (offsets, not a choice between pointers,
  // keep the address arithmetic in registers)
  const uint64_t knew_off = (uint64_t)kncol - (uint64_t)kcol, vnew_off = (uint64_t)vncol - (uint64_t)vcol;
  const int32_t* trow = a.table + w.row * a.stride;
  const int sh = a.page_shift;
  const uint32_t npages = (uint32_t)(a.pool_slots >> sh);
  auto lkey = [&](int r) { return lkey0 + r * NW * KPB; };
  int32_t slot[2][KPT];

  // slots of this lane's keys in the stage starting at kt (pool keys only)
  // Branch-free and never read here: every lane loads a table entry the row
  // holds (a key past the prefix loads a dummy one, ignored when the loads
  // are issued), so no wait for these loads lands before their use a stage
  // later.
  auto load_slots = [&](int (&sl)[KPT], int kt) {
    if (kt >= w.ext_begin) return;  // (uniform) only new tokens: no table entries needed
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int j = min(kt + lkey(r), w.key_end - 1);  // keys past the end repeat the last one
      sl[r] = trow[max(min(j, w.ext_begin - 1), 0) >> sh];  // raw entry: converted when issued
    }
  };
  int bad_slot = 0;  // an out-of-range slot was met (reported once, at the end)
  // The loads are written as assembly.  Issued through the compiler builtin,
  // the compiler cannot tell their LDS writes (the next stage's buffer) from
  // the tile being read, and waits for all of them before the stage's first
  // LDS read, which puts the full load latency into every stage.  Hidden from
  // the compiler, they are ordered by the stage loop alone: each stage waits
  // for its own loads (vmcnt(0)) before the barrier that precedes any read of
  // the buffer they fill.  M0 holds the LDS destination; one wait state
  // separates its write from the load that reads it.
  auto dma = [&](const char* src, uint16_t* dst) {
    const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)dst;
    if constexpr (STREAM)
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(src), "s"(lds) : "memory", "m0");
    else
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "memory", "m0");
  };
  // this lane's 16 bytes of a 1 KiB block, as a load would have written them
  auto zero16 = [&](uint16_t* dst) { *(u32x4*)(dst + lane * 8) = u32x4{0, 0, 0, 0}; };
  // Out-of-range slots are clamped (and reported), so every load stays in
  // the pool; the careful pass stores zeros for them instead.  Keys past the
  // range end are loaded as copies of the last key, so the tile holds finite
  // values where p = 0 multiplies them.
  auto issue = [&](uint16_t* dk, uint16_t* dv, const int (&sl)[KPT], int kt) {
    if (kt + BN <= plain_end) {  // every key of the stage is a cached prefix key
      uint32_t s[KPT], mx = 0;
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        s[r] = (uint32_t)page_slot(sl[r], kt + lkey(r), sh, npages);
        mx = max(mx, s[r]);
      }
      bad_slot |= mx >= nslots;
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        const uint64_t off = (uint64_t)min(s[r], nslots - 1) * row_bytes;
        const int blk = (NW * r + wave) * KPB * D;
        if (CAREFUL && s[r] >= nslots) {
          zero16(dk + blk);
          zero16(dv + blk);
        } else {
          dma(kcol + off, dk + blk);
          dma(vcol + off, dv + blk);
        }
      }
      return;
    }
    if (kt >= w.ext_begin) {  // every key of the stage is a new token
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        const int blk = (NW * r + wave) * KPB * D;
        const uint64_t off = (uint64_t)(w.ext_base + (min(kt + lkey(r), w.key_end - 1) - w.ext_begin)) * row_bytes;
        dma(kncol + off, dk + blk);
        dma(vncol + off, dv + blk);
      }
      return;
    }
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int blk = (NW * r + wave) * KPB * D;
      const int j = min(kt + lkey(r), w.key_end - 1);
      const bool is_new = j >= w.ext_begin;
      const uint32_t sr = (uint32_t)page_slot(sl[r], j, sh, npages);
      bad_slot |= !is_new && sr >= nslots;
      const uint64_t idx = is_new ? (uint64_t)(w.ext_base + (j - w.ext_begin)) : (uint64_t)min(sr, nslots - 1);
      const uint64_t kb_ = (uint64_t)kcol + (is_new ? knew_off : 0);
      const uint64_t vb_ = (uint64_t)vcol + (is_new ? vnew_off : 0);
      if (CAREFUL && !is_new && sr >= nslots) {
        zero16(dk + blk);
        zero16(dv + blk);
      } else {
        dma((const char*)(kb_ + idx * row_bytes), dk + blk);
        dma((const char*)(vb_ + idx * row_bytes), dv + blk);
      }
    }
  };
  // careful pass: is key j (a pool key below the range end) without a valid slot?
  auto absent = [&](int j) {
    return j < plain_end && (uint32_t)page_slot(trow[j >> sh], j, sh, npages) >= nslots;
  };

  // S^T for the two 32-key halves of the stage in LDS.  The halves' MFMA
  // chains interleave; the issue order is pinned (sched_group_barrier) so
  // the K fragment reads run three k-steps ahead of the MFMAs that use them
  // (the compiler otherwise reads each fragment just before its MFMA).
  auto qk = [&](const uint16_t* tk, f32x16& s0, f32x16& s1) {
    s0 = f32x16{};
    s1 = f32x16{};
    const int key = lane & 31;
    const uint16_t* row0 = tk + key * D;
    const uint16_t* row1 = tk + (32 + key) * D;
    const int sw = swz<D>(key);  // the same for key + 32
    bf16x8 k0[NKS], k1[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int ch = ((2 * ks + hi) ^ sw) << 3;
      k0[ks] = *(const bf16x8*)(row0 + ch);
      k1[ks] = *(const bf16x8*)(row1 + ch);
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0[ks], qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1[ks], qf[ks], s1, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < NKS - 3; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
  };
  // Online softmax over the stage's 64 keys (masked on boundary stages only):
  // one maximum per column per stage, the cross-half exchange by a lane swap
  auto softmax = [&](f32x16& s0, f32x16& s1, int kt, auto maskc, bf16x8 (&pf)[4]) {
    constexpr bool MASK = decltype(maskc)::value;
    if constexpr (MASK) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kt + (v >> 2) * 8 + hi * 4 + (v & 3);
        s0[v] = (key >= w.key_end || key > col.limit) ? -INFINITY : s0[v];
        s1[v] = (key + 32 >= w.key_end || key + 32 > col.limit) ? -INFINITY : s1[v];
        if constexpr (CAREFUL) {
          s0[v] = absent(key) ? -INFINITY : s0[v];
          s1[v] = absent(key + 32) ? -INFINITY : s1[v];
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(fmaxf(mx, s0[v]), s1[v]);  // one v_max3 per pair
    const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mx), __builtin_bit_cast(uint32_t, mx),
                                                     false, false);
    mx = fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1])) * a.scale_log2;
    const bool upd = mx > m_run + RESCALE_SLACK;
    if (__any(upd)) {
      const float m_new = upd ? mx : m_run;
      const float alpha = upd ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      s0[v] = __builtin_amdgcn_exp2f(fmaf(s0[v], a.scale_log2, -m_use));
      s1[v] = __builtin_amdgcn_exp2f(fmaf(s1[v], a.scale_log2, -m_use));
    }
    // P rounded to bf16 once: the PV operands, and (two keys per v_dot2 with
    // ones) the denominator, so numerator and denominator use the same weights
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pf[0][i] = (__bf16)s0[i];
      pf[1][i] = (__bf16)s0[8 + i];
      pf[2][i] = (__bf16)s1[i];
      pf[3][i] = (__bf16)s1[8 + i];
    }
    const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ps[k2] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[k2][2 * j], pf[k2][2 * j + 1]}, one2, ps[k2], false);
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
  };
  // O^T += V^T P^T for half h (two 16-key steps); V^T by transposing reads
  auto pv = [&](const bf16x8 (&pfs)[4], const uint16_t* tv, int h) {
    const int g = lane >> 4, r = lane & 15;
    const int dsub = 16 * (g & 1) + 4 * (r & 3);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int k2 = 2 * h + hh;
      const bf16x8 pf = pfs[k2];
      const int key0 = 16 * k2 + 4 * (g >> 1) + (r >> 2);
      const int key1 = key0 + 8;
      const int sw0 = swz<D>(key0), sw1 = swz<D>(key1);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = db * 32 + dsub;
        const i16x4 lo = lds_read_tr(tv + key0 * D + (((d >> 3) ^ sw0) << 3) + (d & 7));
        const i16x4 up = lds_read_tr(tv + key1 * D + (((d >> 3) ^ sw1) << 3) + (d & 7));
        const i16x8 both = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), pf, acc[db], 0, 0, 0);
      }
    }
  };
  auto compute = [&](const uint16_t* tk, const uint16_t* tv, int kt, auto maskc) {
    f32x16 s0, s1;
    bf16x8 pf[4];
    qk(tk, s0, s1);
    softmax(s0, s1, kt, maskc, pf);
    pv(pf, tv, 0);
    pv(pf, tv, 1);
  };

  // Pipeline: LDS double buffer.  At each stage's barrier the stage's tile has
  // landed (every wave waited for its own loads) and the other buffer's reads
  // are done; the next stage's loads then fly while this one is computed, and
  // slot indices run one stage further ahead.
  const int kb = w.key_begin;
  const int n_st = (w.key_end - kb + BN - 1) / BN;
  if (n_st > 0) load_slots(slot[0], kb);
  if (n_st > 1) load_slots(slot[1], kb + BN);
  if (n_st > 0) issue(sK[0], sV[0], slot[0], kb);

  auto step = [&](auto bufc, int i, auto maskc) {
    constexpr int b = decltype(bufc)::value;
    const int kt = kb + i * BN;
    // vmcnt(0) through the builtin, so the compiler knows every earlier load
    // (the slot indices among them) has landed and adds no waits of its own
    // that would also count the assembly loads in flight
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (i + 1 < n_st) issue(sK[b ^ 1], sV[b ^ 1], slot[b ^ 1], kt + BN);
    if (i + 2 < n_st) load_slots(slot[b], kt + 2 * BN);
    if (active) compute(sK[b], sV[b], kt, maskc);
  };
  // stages before n_plain need no mask: every key is below the range end and
  // at or below every column's causal limit; the rest (a tail) are masked
  int n_plain = CAREFUL ? 0 : (w.key_end - kb) / BN;
  if (w.min_limit != INT_MAX) n_plain = min(n_plain, max(0, (w.min_limit + 1 - kb) / BN));
  const auto B0 = std::integral_constant<int, 0>{};
  const auto B1 = std::integral_constant<int, 1>{};
  int i = 0;
  for (; i + 1 < n_plain; i += 2) {
    step(B0, i, std::false_type{});
    step(B1, i + 1, std::false_type{});
  }
  if (i < n_plain) {
    step(B0, i, std::false_type{});
    ++i;
    if (i < n_st) {
      step(B1, i, std::true_type{});
      ++i;
    }
  }
  for (; i < n_st; i += 2) {
    step(B0, i, std::true_type{});
    if (i + 1 < n_st) step(B1, i + 1, std::true_type{});
  }

  if constexpr (!CAREFUL) {
    if (bad_slot) s_absent = 1;
    __syncthreads();
    if (s_absent) {  // some key is absent: the careful pass computes the item
      if (threadIdx.x == 0) flag(a.err, RC_DEVERR_SLOT);
      return true;
    }
  }
  if (!active || !col.real) return false;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (mode == EXTEND) {
    const float inv = 1.f / l_tot;
    {
      uint16_t* o = (uint16_t*)a.o + col.qoff * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + g4 * 8 + hi * 4;
          __bf16 b0 = (__bf16)(acc[db][4 * g4 + 0] * inv), b1 = (__bf16)(acc[db][4 * g4 + 1] * inv);
          __bf16 b2 = (__bf16)(acc[db][4 * g4 + 2] * inv), b3 = (__bf16)(acc[db][4 * g4 + 3] * inv);
          uint2 pk;
          pk.x = pack2(__builtin_bit_cast(uint16_t, b0), __builtin_bit_cast(uint16_t, b1));
          pk.y = pack2(__builtin_bit_cast(uint16_t, b2), __builtin_bit_cast(uint16_t, b3));
          *(uint2*)(o + d) = pk;
        }
    }
  } else {
    // the partial row normalised by its own sum and rounded to bf16 once; the
    // merge weighs the rows by their (max, sum) pairs in fp32
    const int64_t pidx = ((int64_t)col.b * a.Hq + col.head) * a.max_splits + w.split;
    uint16_t* wo = (uint16_t*)a.ws_o + pidx * D;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + hi * 4;
        const __bf16 b0 = (__bf16)(acc[db][4 * g4 + 0] * inv), b1 = (__bf16)(acc[db][4 * g4 + 1] * inv);
        const __bf16 b2 = (__bf16)(acc[db][4 * g4 + 2] * inv), b3 = (__bf16)(acc[db][4 * g4 + 3] * inv);
        uint2 pk;
        pk.x = pack2(__builtin_bit_cast(uint16_t, b0), __builtin_bit_cast(uint16_t, b1));
        pk.y = pack2(__builtin_bit_cast(uint16_t, b2), __builtin_bit_cast(uint16_t, b3));
        *(uint2*)(wo + d) = pk;
      }
    if (hi == 0) *(float2*)(a.ws_ml + pidx * 2) = make_float2(m_run, l_tot);
  }
  return false;
}

// One MFMA work item: the usual pass, then the careful one if a key was absent.
template <int D, int NW, bool STREAM>
__device__ __forceinline__ void attn_bf16_tile(const Args& a, const int mode, const int L, uint16_t (&sK)[2][BN * D],
                                               uint16_t (&sV)[2][BN * D]) {
  if (attn_bf16_body<D, NW, STREAM, false>(a, mode, L, sK, sV)) attn_bf16_body<D, NW, STREAM, true>(a, mode, L, sK, sV);
}

// fp32 path: one wave per column; its 64 lanes are 16 keys x 4 groups of
// D/4 head dims, so a wave takes 16 keys at a time: each lane dots its key's
// group with the query's (two shuffles finish the score), the online softmax
// moves once per 16 keys, and each lane accumulates p x V for its key and
// group; the 16 key lanes of each group are summed once, at the end.  Same
// work decomposition and outputs as the MFMA kernel; used for fp32 data.
template <int D>
__device__ __forceinline__ void attn_f32_body(const Args& a, const int mode) {
  constexpr int DG = D / 4;     // head dims per lane group
  constexpr int NV = DG / 4;    // float4 per lane and row
  const int L = xcd_remap(blockIdx.x, a.n_work);
  const Work w = resolve(a, mode, L, threadIdx.x == 0);
  if (!w.valid) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kk = lane >> 2, grp = lane & 3;  // key within the 16, head-dim group
  if (w.store_b >= 0) store_new_token<float, D>(a, w.store_b, w.hk, threadIdx.x);
  const float* q = (const float*)a.q;
  const float* kpool = (const float*)a.k_pool;
  const float* vpool = (const float*)a.v_pool;
  const float* knew = (const float*)a.k_new;
  const float* vnew = (const float*)a.v_new;
  const int64_t rowHD = (int64_t)a.Hkv * D;
  const int64_t head_off = (int64_t)w.hk * D + grp * DG;
  const uint32_t npages = (uint32_t)(a.pool_slots >> a.page_shift);
  // row offset (in floats, from the pool or from k_new/v_new) of key j; -1: no key
  auto row_of = [&](int j, int end, bool& from_new) -> int64_t {
    from_new = false;
    if (j >= end) return -1;
    if (j >= w.ext_begin) {
      from_new = true;
      return (w.ext_base + (j - w.ext_begin)) * rowHD + head_off;
    }
    const int32_t sl = page_slot(a.table[w.row * a.stride + (j >> a.page_shift)], j, a.page_shift, npages);
    if (sl < 0 || (int64_t)sl >= a.pool_slots) {
      if (grp == 0) flag(a.err, RC_DEVERR_SLOT);  // an absent key
      return -1;
    }
    return (int64_t)sl * rowHD + head_off;
  };
  for (int c = wave; c < w.ncols; c += NT / 64) {
    const Col col = column(a, mode, w, c);
    float4 qv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) qv[i] = *(const float4*)(q + col.qoff * D + grp * DG + 4 * i);
    float4 ov[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) ov[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    float m_run = -INFINITY, l_run = 0.f;
    const int end = min(w.key_end, col.limit == INT_MAX ? w.key_end : col.limit + 1);
    for (int j0 = w.key_begin; j0 < end; j0 += 16) {
      bool from_new;
      const int64_t off = row_of(j0 + kk, end, from_new);
      const bool has = off >= 0;
      const float* kp = (from_new ? knew : kpool) + (has ? off : 0);
      const float* vp = (from_new ? vnew : vpool) + (has ? off : 0);
      float4 kv[NV], vv[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        kv[i] = has ? *(const float4*)(kp + 4 * i) : make_float4(0.f, 0.f, 0.f, 0.f);
        vv[i] = has ? *(const float4*)(vp + 4 * i) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < NV; ++i) dot += qv[i].x * kv[i].x + qv[i].y * kv[i].y + qv[i].z * kv[i].z + qv[i].w * kv[i].w;
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
      const float x = has ? dot * a.scale_log2 : -INFINITY;
      float mx = x;
#pragma unroll
      for (int sh = 4; sh <= 32; sh <<= 1) mx = fmaxf(mx, __shfl_xor(mx, sh));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      const float pr = has ? exp2f(x - m_use) : 0.f;
      l_run = l_run * alpha + pr;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        ov[i].x = ov[i].x * alpha + pr * vv[i].x;
        ov[i].y = ov[i].y * alpha + pr * vv[i].y;
        ov[i].z = ov[i].z * alpha + pr * vv[i].z;
        ov[i].w = ov[i].w * alpha + pr * vv[i].w;
      }
      m_run = m_new;
    }
    // sum over the 16 key lanes of each head-dim group
#pragma unroll
    for (int sh = 4; sh <= 32; sh <<= 1) {
      l_run += __shfl_xor(l_run, sh);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        ov[i].x += __shfl_xor(ov[i].x, sh);
        ov[i].y += __shfl_xor(ov[i].y, sh);
        ov[i].z += __shfl_xor(ov[i].z, sh);
        ov[i].w += __shfl_xor(ov[i].w, sh);
      }
    }
    if (!col.real || kk != 0) continue;
    if (mode == EXTEND) {
      float* o = (float*)a.o + col.qoff * D + grp * DG;
      const float inv = 1.f / l_run;
#pragma unroll
      for (int i = 0; i < NV; ++i) *(float4*)(o + 4 * i) = make_float4(ov[i].x * inv, ov[i].y * inv, ov[i].z * inv, ov[i].w * inv);
    } else {
      const int64_t pidx = ((int64_t)col.b * a.Hq + col.head) * a.max_splits + w.split;
#pragma unroll
      for (int i = 0; i < NV; ++i) *(float4*)((float*)a.ws_o + pidx * D + grp * DG + 4 * i) = ov[i];
      if (grp == 0) *(float2*)(a.ws_ml + pidx * 2) = make_float2(m_run, l_run);
    }
  }
}

rc_status check_common(const rc_shape* shape, float sm_scale) {
  rc_status st = rc::check_shape(shape);
  if (st != RC_OK) return st;
  // the kernels take each column's maximum over raw scores and scale it after
  // (exact for a positive scale), and masked keys hold -inf scores
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.f))
    return rc::fail(RC_ERR_ARG, "sm_scale %g is not a finite positive number", (double)sm_scale);
  return RC_OK;
}

}  // namespace
