// Split-K decode attention over a shared plan: one query token per request
// attends over its whole context; shared tree ranges are read once for all
// the requests that pass through them.
#include <mutex>

#include "attn_tile.h"

namespace {

// Narrow decode items (members x group <= 16 query columns): one wave per
// (item, kv head), no workgroup barriers.  Per 32-key stage a lane loads 8
// keys' K and V chunks with 16 lanes per key row, so every load instruction
// moves 4 keys x 256 contiguous bytes (gathers that scatter an instruction over
// 16 slots reach only about half the bandwidth); the stage goes into a
// wave-private row-major LDS tile (chunk-swizzled per key), from which the
// K operand is read with ds_read_b128 and V^T with transposing reads.  The
// next stage's K and V are in registers while this one is computed; slot
// indices run one more stage ahead.  S^T = K Q^T and O^T += V^T P^T on
// v_mfma_f32_16x16x32_bf16 tiles: a lane owns one query column and 4 keys per
// 16-key block, so the softmax reductions cross the 4 lane groups (2 steps).
constexpr int BNN = 32;  // keys per narrow stage

// STREAM: nontemporal K/V loads (see attn_bf16_body).  CAREFUL: the second
// pass over an item that met a key without a valid slot (as in attn_bf16_body):
// the usual pass returns true without writing, the careful one loads zeros for
// such keys and gives them a -inf score.
template <int D, bool STREAM = false, bool CAREFUL = false>
__device__ __forceinline__ bool decode_narrow_body(const Args& a, const int unit, uint16_t* sk, uint16_t* sv) {
  constexpr int NKS = D / 32;         // k-steps of 32 over D
  constexpr int NDB = D / 16;         // 16-row blocks of O^T
  constexpr int CH = D / 8;           // 16-byte chunks per key row
  constexpr int KPI = 64 / CH;        // keys per load instruction (4 for D=128, 8 for D=64)
  constexpr int NI = BNN / KPI;       // load instructions per lane per stage and array
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, r16 = lane & 15;
  const int L = (a.narrow_begin + unit / a.Hkv) * a.Hkv + unit % a.Hkv;
  const Work w = resolve(a, DECODE, L, lane == 0);
  if (!w.valid) return false;  // uniform over the wave
  const Col col = column(a, DECODE, w, r16);

  const uint16_t* q = (const uint16_t*)a.q;
  bf16x8 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8*)(q + col.qoff * D + ks * 32 + 8 * grp);

  f32x4 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;

  const int lc = lane % CH, lk = lane / CH;  // loader: chunk and key within an instruction
  const uint16_t* kbase = (const uint16_t*)a.k_pool + (int64_t)w.hk * D + lc * 8;
  const uint16_t* vbase = (const uint16_t*)a.v_pool + (int64_t)w.hk * D + lc * 8;
  const int64_t rowHD = (int64_t)a.Hkv * D;
  const int32_t* trow = a.table + w.row * a.stride;
  const int sh = a.page_shift;
  const uint32_t npages = (uint32_t)(a.pool_slots >> sh);
  int bad_slot = 0;

  constexpr int NEWTOK = INT_MIN + 1;  // the current token: read from k_new/v_new
  // raw table entries, converted to slots when the stage's K/V are loaded
  auto load_slots = [&](int (&sl)[NI], int kt) {
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      const int key = kt + t * KPI + lk;
      // INT_MIN: past the range end
      sl[t] = key < w.key_end ? (key >= w.ext_begin ? NEWTOK : trow[key >> sh]) : INT_MIN;
    }
  };
  // careful pass: bit k of the stage's mask marks key kt + k as absent (set
  // when the stage is loaded, from a ballot of the lanes that load the key)
  uint32_t absent_next = 0, absent_cur = 0;
  auto load_kv = [&](u32x4 (&kr)[NI], u32x4 (&vr)[NI], const int (&sl)[NI], int kt, bool partial) {
    if constexpr (CAREFUL) absent_next = 0;
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      const bool special = sl[t] == INT_MIN || sl[t] == NEWTOK;
      const int32_t st = special ? sl[t] : page_slot(sl[t], kt + t * KPI + lk, sh, npages);
      const bool ok = (uint32_t)st < (uint32_t)a.pool_slots;
      bad_slot |= !ok & !special;
      if constexpr (CAREFUL) {
        const uint64_t bl = __ballot(!ok & !special);  // lane lk * CH loads key t * KPI + lk's first chunk
#pragma unroll
        for (int k = 0; k < KPI; ++k) absent_next |= (uint32_t)((bl >> (k * CH)) & 1) << (t * KPI + k);
      }
      const int64_t off = (int64_t)(ok ? st : 0) * rowHD;
      if constexpr (STREAM) {
        kr[t] = __builtin_nontemporal_load((const u32x4*)(kbase + off));
        vr[t] = __builtin_nontemporal_load((const u32x4*)(vbase + off));
      } else {
        kr[t] = *(const u32x4*)(kbase + off);
        vr[t] = *(const u32x4*)(vbase + off);
      }
      if (partial && !ok) {  // keys past the end must hold finite values: p = 0 multiplies them
        kr[t] = u32x4{0, 0, 0, 0};
        vr[t] = u32x4{0, 0, 0, 0};
        if (st == NEWTOK) {
          const int64_t noff = ((int64_t)w.ext_base * a.Hkv + w.hk) * D + lc * 8;
          kr[t] = *(const u32x4*)((const uint16_t*)a.k_new + noff);
          vr[t] = *(const u32x4*)((const uint16_t*)a.v_new + noff);
        }
      }
    }
  };
  // (the careful pass stores zeros for absent keys: they were loaded from a
  // stand-in slot, and p = 0 multiplies them)
  auto store = [&](const u32x4 (&kr)[NI], const u32x4 (&vr)[NI]) {
    if constexpr (CAREFUL) absent_cur = absent_next;
#pragma unroll
    for (int t = 0; t < NI; ++t) {
      const int key = t * KPI + lk;
      const int o = key * D + ((lc ^ swz<D>(key)) << 3);
      const bool z = CAREFUL && ((absent_cur >> key) & 1);
      *(u32x4*)(sk + o) = z ? u32x4{0, 0, 0, 0} : kr[t];
      *(u32x4*)(sv + o) = z ? u32x4{0, 0, 0, 0} : vr[t];
    }
  };
  auto compute = [&](int kt) {
    f32x4 s[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      s[j] = f32x4{};
      const int key = 16 * j + r16;
      const int sw = swz<D>(key);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 kf = *(const bf16x8*)(sk + key * D + (((4 * ks + grp) ^ sw) << 3));
        s[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], s[j], 0, 0, 0);
      }
    }
    const bool need_mask = kt + BNN > w.key_end;
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key = kt + 16 * j + 4 * grp + v;
        float x = s[j][v];
        if (need_mask && key >= w.key_end) x = -INFINITY;
        if (CAREFUL && ((absent_cur >> (key - kt)) & 1)) x = -INFINITY;  // a key without a valid slot
        s[j][v] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.scale_log2;
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[j][v], a.scale_log2, -m_use));
        s[j][v] = p;
        psum += p;
      }
    if (__any(m_new != m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    }
    l_run += psum;
    m_run = m_new;
    // P^T operand: k-position 8*grp+i <-> key 16*(i/4) + 4*grp + i%4
    bf16x8 pf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pf[i] = (__bf16)s[0][i];
      pf[4 + i] = (__bf16)s[1][i];
    }
    const int key0 = 4 * grp + (r16 >> 2), key1 = key0 + 16;
    const int sw0 = swz<D>(key0), sw1 = swz<D>(key1);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = db * 16 + 4 * (r16 & 3);
      const i16x4 lo = lds_read_tr(sv + key0 * D + (((d >> 3) ^ sw0) << 3) + (d & 7));
      const i16x4 up = lds_read_tr(sv + key1 * D + (((d >> 3) ^ sw1) << 3) + (d & 7));
      const i16x8 both = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, both), pf, acc[db], 0, 0, 0);
    }
  };

  if (w.store_b >= 0) store_new_token<uint16_t, D>(a, w.store_b, w.hk, lane);
  const int kb = w.key_begin;
  const int n_st = (w.key_end - kb + BNN - 1) / BNN;
  const int plain_end = min(w.key_end, w.ext_begin);  // stages ending after this take the careful path
  int slA[NI], slB[NI];
  u32x4 kr[NI], vr[NI];
  if constexpr (CAREFUL) {
    // the careful pass runs its stages one after the other (no prefetch)
    for (int i = 0; i < n_st; ++i) {
      const int kt = kb + i * BNN;
      load_slots(slA, kt);
      load_kv(kr, vr, slA, kt, true);
      store(kr, vr);
      compute(kt);
    }
  }
  if (!CAREFUL && n_st > 0) load_slots(slA, kb);
  if (!CAREFUL && n_st > 1) load_slots(slB, kb + BNN);
  if (!CAREFUL && n_st > 0) load_kv(kr, vr, slA, kb, kb + BNN > plain_end);
  if (!CAREFUL && n_st > 2) load_slots(slA, kb + 2 * BNN);
  // The LDS tile is private to the wave and LDS operations of a wave complete
  // in order, so the next stage may overwrite it right after this stage's reads.
  for (int i = 0; !CAREFUL && i < n_st; i += 2) {
    int kt = kb + i * BNN;
    store(kr, vr);
    if (i + 1 < n_st) {
      load_kv(kr, vr, slB, kt + BNN, kt + 2 * BNN > plain_end);
      if (i + 3 < n_st) load_slots(slB, kt + 3 * BNN);
    }
    compute(kt);
    if (i + 1 >= n_st) break;
    kt += BNN;
    store(kr, vr);
    if (i + 2 < n_st) {
      load_kv(kr, vr, slA, kt + BNN, kt + 2 * BNN > plain_end);
      if (i + 4 < n_st) load_slots(slA, kt + 3 * BNN);
    }
    compute(kt);
  }

  if constexpr (!CAREFUL) {
    if (__any(bad_slot)) {  // some key is absent: the careful pass computes the item
      if (lane == 0) flag(a.err, RC_DEVERR_SLOT);
      return true;
    }
  }
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!col.real) return false;
  const int64_t pidx = ((int64_t)col.b * a.Hq + col.head) * a.max_splits + w.split;
  uint16_t* wo = (uint16_t*)a.ws_o + pidx * D;  // the normalised partial row in bf16, as in the wide tile
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    uint2 pk;
    pk.x = pack2(__builtin_bit_cast(uint16_t, (__bf16)(acc[db][0] * inv)), __builtin_bit_cast(uint16_t, (__bf16)(acc[db][1] * inv)));
    pk.y = pack2(__builtin_bit_cast(uint16_t, (__bf16)(acc[db][2] * inv)), __builtin_bit_cast(uint16_t, (__bf16)(acc[db][3] * inv)));
    *(uint2*)(wo + db * 16 + 4 * grp) = pk;
  }
  if (grp == 0) *(float2*)(a.ws_ml + pidx * 2) = make_float2(m_run, l_tot);
  return false;
}

// Decode, one launch: the plan lists wide items (workgroup-cooperative tiles,
// heaviest first) before narrow ones, and blocks are dispatched in order, so
// the long wide workgroups start first and the narrow ones (four independent
// waves per block, each with its own K and V tile) fill in behind them.  Both
// paths need 2 waves per SIMD and 64 KiB of LDS, so one kernel costs neither
// occupancy, and there is no gap between two launches.  ROLE 0: decode steps,
// whose K/V loads are nontemporal (each range is read once per launch: 8 % faster
// on the heavy-decode workload); ROLE 1: extends run over a shared-prefix plan
// (the members are new tokens), whose member groups re-read a prompt and keep
// it in L2.  The two instantiations also tell the paths apart in profiles.
// Decode steps take four-wave workgroups (two per CU); the cascade extend
// takes eight-wave ones (one per CU), whose wide items carry up to
// RC_EXTEND_SHARED_COLS query columns, so each K/V stage loaded into LDS feeds
// twice the columns, as in the extend tile.
template <int ROLE>
constexpr int role_waves() {
  return ROLE == 0 ? 4 : 8;
}

template <int D, int ROLE>
__global__ __launch_bounds__(64 * role_waves<ROLE>(), ROLE == 0 ? 2 : 1) void decode_attn_bf16(Args a) {
  constexpr int NWK = role_waves<ROLE>();
  // 64-key blocks: the wide tile's two K and two V stages use the first two,
  // the narrow waves' 32-key tiles all of them
  constexpr int NB = NWK * BNN / BN;
  static_assert(NB >= 2 && NB * BN == NWK * BNN, "narrow tiles and wide stages share the buffers");
  __shared__ __attribute__((aligned(16))) uint16_t sK[NB][BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[NB][BN * D];
  // the grid is [wide workgroups][narrow workgroups], or the other way round
  // when the plan says the narrow class runs longer (workgroups start in order)
  const int n_narrow_blocks = (a.n_narrow_units + NWK - 1) / NWK;
  const int bid = (int)blockIdx.x;
  const bool wide = a.narrow_first ? bid >= n_narrow_blocks : bid < a.n_wide_blocks;
  if (wide) {
    typedef uint16_t Stages[2][BN * D];
    attn_bf16_tile<D, NWK, ROLE == 0>(a, DECODE, a.narrow_first ? bid - n_narrow_blocks : bid,
                                      *reinterpret_cast<Stages*>(&sK[0][0]), *reinterpret_cast<Stages*>(&sV[0][0]));
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int unit = (a.narrow_first ? bid : bid - a.n_wide_blocks) * NWK + wave;
  if (unit >= a.n_narrow_units) return;
  uint16_t* sk = &sK[0][0] + wave * BNN * D;
  uint16_t* sv = &sV[0][0] + wave * BNN * D;
  if (decode_narrow_body<D, ROLE == 0, false>(a, unit, sk, sv)) decode_narrow_body<D, ROLE == 0, true>(a, unit, sk, sv);
}

template <int D>
__global__ __launch_bounds__(NT) void decode_attn_f32(Args a) {
  attn_f32_body<D>(a, DECODE);
}

// Split merge: for each (request, q head), combine its partials k = 0..n-1 in
// order: M = max m_k, l = sum l_k 2^(m_k - M), o = sum o_k 2^(m_k - M) / l.
// 16 lanes per (request, head), four pairs per wave; a lane handles D/16
// consecutive elements of a row (one 16-byte load per partial row for bf16
// data at D = 128).  The (max, sum) pairs of 16 splits at a time are loaded
// at once (one per lane) and reduced across the 16 lanes; the partial rows are
// then read four at a time with their loads in flight together.  Beyond 16
// splits the blocks are combined with the usual rescaling.  BF16: bf16 data,
// whose partial rows come normalised (o_k / l_k) in bf16, so each row is
// weighed by u_k = l_k 2^(m_k - M) and the same u_k sum to l (with V = 1 the
// output is exactly 1); fp32 data: unnormalised fp32 rows weighed by
// 2^(m_k - M).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void merge_kernel(void* out, const void* __restrict__ ws_o,
                                                    const float* __restrict__ ws_ml, const int32_t* nsplit,
                                                    int32_t batch, int32_t Hq, int32_t max_splits) {
  constexpr int PER = D / 16;
  constexpr int MU = 4;  // partial rows in flight per lane
  typedef __bf16 bvec __attribute__((ext_vector_type(PER)));  // one lane's elements of a bf16 row
  const int lane = threadIdx.x & 63;
  const int sub = lane & 15, gbase = lane & 48;
  const int pair = (int)blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool live = pair < batch * Hq;
  int ns = live ? nsplit[pair / Hq] : 0;
  ns = ns < 0 ? 0 : (ns < max_splits ? ns : max_splits);
  const float* ml = ws_ml + (int64_t)pair * max_splits * 2;
  const int64_t row0 = (int64_t)pair * max_splits * D + sub * PER;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float l = 0.f, M_run = -INFINITY;
  for (int k0 = 0; k0 < ns; k0 += 16) {
    const int k = k0 + sub;
    const float2 mine = k < ns ? *(const float2*)(ml + 2 * k) : make_float2(-INFINITY, 0.f);
    float Mb = mine.x;
#pragma unroll
    for (int sh = 8; sh >= 1; sh >>= 1) Mb = fmaxf(Mb, __shfl_xor(Mb, sh));
    const float M = fmaxf(M_run, Mb);
    if (k0 > 0 && M_run != M) {
      const float r = M_run == -INFINITY ? 0.f : exp2f(M_run - M);
      l *= r;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] *= r;
    }
    M_run = M;
    const float wk = mine.x == -INFINITY ? 0.f : exp2f(mine.x - M);
    const int n = min(16, ns - k0);
    // MU partial rows at a time, their loads issued together (a split past n
    // re-reads the block's last row and gets weight 0)
    for (int j0 = 0; j0 < n; j0 += MU) {
      float wq[MU], uq[MU];
      int64_t eq[MU];
#pragma unroll
      for (int t = 0; t < MU; ++t) {
        const int j = min(j0 + t, n - 1);
        const float wj = __shfl(wk, gbase + j);
        const float uj = __shfl(mine.y, gbase + j) * wj;
        wq[t] = j0 + t < n ? wj : 0.f;
        uq[t] = j0 + t < n ? uj : 0.f;
        eq[t] = row0 + (int64_t)(k0 + j) * D;
      }
      if constexpr (BF16) {
        bvec v[MU];
#pragma unroll
        for (int t = 0; t < MU; ++t) v[t] = *(const bvec*)((const __bf16*)ws_o + eq[t]);
#pragma unroll
        for (int t = 0; t < MU; ++t) {
          l += uq[t];
#pragma unroll
          for (int i = 0; i < PER; ++i) acc[i] += (float)v[t][i] * uq[t];
        }
      } else {
        float4 v[MU][PER / 4];
#pragma unroll
        for (int t = 0; t < MU; ++t)
#pragma unroll
          for (int i = 0; i < PER / 4; ++i) v[t][i] = *(const float4*)((const float*)ws_o + eq[t] + 4 * i);
#pragma unroll
        for (int t = 0; t < MU; ++t) {
          l += uq[t];
#pragma unroll
          for (int i = 0; i < PER / 4; ++i) {
            acc[4 * i] += v[t][i].x * wq[t];
            acc[4 * i + 1] += v[t][i].y * wq[t];
            acc[4 * i + 2] += v[t][i].z * wq[t];
            acc[4 * i + 3] += v[t][i].w * wq[t];
          }
        }
      }
    }
  }
  if (!live) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t o0 = (int64_t)pair * D + sub * PER;
  if constexpr (BF16) {
    bvec r;
#pragma unroll
    for (int i = 0; i < PER; ++i) r[i] = (__bf16)(acc[i] * inv);
    *(bvec*)((__bf16*)out + o0) = r;
  } else {
#pragma unroll
    for (int i = 0; i < PER; i += 4)
      *(float4*)((float*)out + o0 + i) = make_float4(acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv);
  }
}

template <int D>
void launch_decode_f32(const Args& a, int n_work, hipStream_t s, const char* name, bool timed) {
  rc::ProfScope p(name, s, timed);
  hipLaunchKernelGGL(decode_attn_f32<D>, dim3(n_work), dim3(NT), 0, s, a);
}

}  // namespace

extern "C" int64_t rc_decode_workspace_bytes(const rc_shape* shape, const rc_plan_info* info) {
  if (!shape || !info || shape->head_dim <= 0) return -1;
  const int64_t parts = (int64_t)info->batch * shape->num_q_heads * (info->max_splits > 0 ? info->max_splits : 1);
  // partial rows in the data type (bf16 or fp32), then fp32 (max, sum) pairs
  const int64_t row_bytes = shape->head_dim * (shape->dtype == RC_BF16 ? 2 : 4);
  return parts * row_bytes + parts * 2 * 4;
}

namespace {

// Split-K attention over a plan, then the merge: the body of
// rc_decode_attention and rc_decode_attention_static (role 0) and of
// rc_extend_attention_shared (role 1).  timed = false: no kernel timing (the
// allocation-free entry point creates no events).
template <int ROLE>
rc_status split_k_attention(const rc_shape* shape, void* o, const void* q, void* k_pool, void* v_pool,
                            const void* k_new, const void* v_new, const int32_t* new_slots,
                            const int32_t* req_to_token, int32_t table_rows, int64_t stride, const int32_t* seq_lens,
                            int32_t batch, const int32_t* plan_dev, const rc_plan_info* info, float sm_scale,
                            void* workspace, int64_t ws_bytes, void* stream, bool timed = true) {
  using namespace rc;
  const bool d128 = shape && shape->head_dim == 128;
  const char* attn_name = ROLE == 0 ? (d128 ? "decode_attention_d128" : "decode_attention_d64")
                                    : (d128 ? "extend_shared_d128" : "extend_shared_d64");
  const char* merge_name = ROLE == 0 ? "decode_merge" : "extend_shared_merge";
  rc_status st = check_common(shape, sm_scale);
  if (st != RC_OK) return st;
  if (batch < 0 || stride <= 0 || table_rows < 0) return fail(RC_ERR_ARG, "batch < 0, stride <= 0 or table_rows < 0");
  if (batch == 0) return RC_OK;
  if (!info) return fail(RC_ERR_ARG, "plan info is NULL");
  if (!o || !q || !k_pool || !v_pool || !req_to_token || !seq_lens || !plan_dev || !workspace)
    return fail(RC_ERR_ARG, "NULL device pointer in the split-K attention call");
  if ((k_new != nullptr) != (v_new != nullptr) || (k_new != nullptr) != (new_slots != nullptr))
    return fail(RC_ERR_ARG, "k_new, v_new and new_slots must be given together");
  const int g = shape->num_q_heads / shape->num_kv_heads;
  if (info->batch != batch) return fail(RC_ERR_ARG, "plan built for batch %d, called with %d", info->batch, batch);
  if (info->group != g) return fail(RC_ERR_SHAPE, "plan built for group %d, shape has %d", info->group, g);
  constexpr int NWK = role_waves<ROLE>();
  if (info->max_cols > 32 * NWK || info->n_items < 0 || info->n_members < 0 || info->max_splits < 1 ||
      info->plan_ints != RC_PLAN_HEADER + (int64_t)info->n_items * RC_PLAN_ITEM + info->n_members + batch)
    return fail(RC_ERR_ARG, "plan summary out of range");
  const int64_t need = rc_decode_workspace_bytes(shape, info);
  if (ws_bytes < need) return fail(RC_ERR_RANGE, "workspace of %lld bytes, %lld needed", (long long)ws_bytes, (long long)need);
  const int64_t parts = (int64_t)batch * shape->num_q_heads * info->max_splits;
  Args a{};
  a.q = q; a.o = o; a.k_pool = k_pool; a.v_pool = v_pool;
  a.k_new = k_new; a.v_new = v_new; a.new_slots = new_slots;
  a.table = req_to_token; a.table_rows = table_rows; a.stride = stride; a.pool_slots = shape->pool_slots;
  a.page_shift = shape->page_size > 1 ? __builtin_ctz((unsigned)shape->page_size) : 0;
  a.Hq = shape->num_q_heads; a.Hkv = shape->num_kv_heads; a.g = g;
  a.scale_log2 = sm_scale * LOG2E;
  a.err = error_word();
  a.batch = batch;
  a.plan = plan_dev; a.seq_lens = seq_lens;
  a.n_items = info->n_items; a.n_members = info->n_members;
  a.narrow_begin = info->narrow_begin;
  a.narrow_first = info->narrow_first != 0;
  a.ws_o = workspace;
  a.ws_ml = (float*)((char*)workspace + parts * shape->head_dim * (shape->dtype == RC_BF16 ? 2 : 4));
  a.max_splits = info->max_splits;
  a.max_cols = 32 * NWK;
  if (info->narrow_begin < 0 || info->narrow_begin > info->n_items) return fail(RC_ERR_ARG, "plan summary out of range");
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = shape->dtype == RC_BF16;
  if (!bf16) {
    const int64_t n_work = (int64_t)info->n_items * a.Hkv;
    if (n_work > INT32_MAX) return fail(RC_ERR_RANGE, "grid too large");
    a.n_work = (int32_t)n_work;
    if (n_work > 0) {
      if (shape->head_dim == 128)
        launch_decode_f32<128>(a, a.n_work, s, "decode_f32_d128", timed);
      else
        launch_decode_f32<64>(a, a.n_work, s, "decode_f32_d64", timed);
      st = check_launch("decode attention");
      if (st != RC_OK) return st;
    }
  } else {
    // wide items: one workgroup per (item, kv head)
    const int64_t n_wide = (int64_t)info->narrow_begin * a.Hkv;
    // narrow items: one wave per (item, kv head), NWK waves per workgroup
    const int64_t units = (int64_t)(info->n_items - info->narrow_begin) * a.Hkv;
    const int64_t n_narrow = (units + NWK - 1) / NWK;
    const int64_t grid = n_wide + n_narrow;
    if (grid > INT32_MAX) return fail(RC_ERR_RANGE, "grid too large");
    a.n_narrow_units = (int32_t)units;
    a.n_wide_blocks = (int32_t)n_wide;
    if (grid > 0) {
      ProfScope p(attn_name, s, timed);
      if (shape->head_dim == 128)
        hipLaunchKernelGGL((decode_attn_bf16<128, ROLE>), dim3((unsigned)grid), dim3(64 * NWK), 0, s, a);
      else
        hipLaunchKernelGGL((decode_attn_bf16<64, ROLE>), dim3((unsigned)grid), dim3(64 * NWK), 0, s, a);
    }
    st = check_launch("decode attention");
    if (st != RC_OK) return st;
  }
  const int32_t* nsplit = plan_dev + RC_PLAN_HEADER + (int64_t)info->n_items * RC_PLAN_ITEM + info->n_members;
  const int pairs = batch * shape->num_q_heads;
  const dim3 grid((pairs + 15) / 16);
  {
    ProfScope p(merge_name, s, timed);
    if (shape->head_dim == 128) {
      if (bf16)
        hipLaunchKernelGGL((merge_kernel<128, true>), grid, dim3(256), 0, s, o, a.ws_o, a.ws_ml, nsplit, batch, a.Hq, a.max_splits);
      else
        hipLaunchKernelGGL((merge_kernel<128, false>), grid, dim3(256), 0, s, o, a.ws_o, a.ws_ml, nsplit, batch, a.Hq, a.max_splits);
    } else {
      if (bf16)
        hipLaunchKernelGGL((merge_kernel<64, true>), grid, dim3(256), 0, s, o, a.ws_o, a.ws_ml, nsplit, batch, a.Hq, a.max_splits);
      else
        hipLaunchKernelGGL((merge_kernel<64, false>), grid, dim3(256), 0, s, o, a.ws_o, a.ws_ml, nsplit, batch, a.Hq, a.max_splits);
    }
  }
  return check_launch("decode merge");
}

}  // namespace

extern "C" rc_status rc_decode_attention(const rc_shape* shape, void* o, const void* q, void* k_pool,
                                         void* v_pool, const void* k_new, const void* v_new,
                                         const int32_t* new_slots, const int32_t* req_to_token, int32_t table_rows,
                                         int64_t stride, const int32_t* seq_lens, int32_t batch, const int32_t* plan_dev,
                                         const rc_plan_info* info, float sm_scale, void* workspace,
                                         int64_t ws_bytes, void* stream) {
  return split_k_attention<0>(shape, o, q, k_pool, v_pool, k_new, v_new, new_slots, req_to_token, table_rows, stride,
                              seq_lens, batch, plan_dev, info, sm_scale, workspace, ws_bytes, stream);
}

// Workspace of rc_decode_attention_static: a file-scope device array, one copy
// per GPU, which the process holds until it ends.  Host code never uses the
// array's name as an address (on the host it is only a stand-in for the
// symbol): each device's address comes from hipGetSymbolAddress, taken once
// per device with that device current, and goes to the kernels as the
// workspace pointer.
static __device__ __align__(256) unsigned char scratch[RC_DECODE_STATIC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's address on the current device.
rc_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return rc::fail(RC_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return rc::fail(RC_ERR_HIP, "device %d beyond the %d this library serves", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return rc::fail(RC_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RC_OK;
}

}  // namespace

extern "C" rc_status rc_decode_attention_static(const rc_shape* shape, void* o, const void* q, void* k_pool,
                                                void* v_pool, const void* k_new, const void* v_new,
                                                const int32_t* new_slots, const int32_t* req_to_token,
                                                int32_t table_rows, int64_t stride, const int32_t* seq_lens,
                                                int32_t batch, const int32_t* plan_dev, const rc_plan_info* info,
                                                float sm_scale, void* stream) {
  if (!shape || !info) return rc::fail(RC_ERR_ARG, "shape or plan info is NULL");
  if (batch == 0) return RC_OK;
  const int64_t need = rc_decode_workspace_bytes(shape, info);
  if (need < 0 || need > RC_DECODE_STATIC_WORKSPACE_BYTES)
    return rc::fail(RC_ERR_RANGE, "the plan needs %lld bytes of workspace, above the %lld of the static workspace",
                    (long long)need, (long long)RC_DECODE_STATIC_WORKSPACE_BYTES);
  void* ws = nullptr;
  rc_status st = scratch_on_current_device(&ws);
  if (st != RC_OK) return st;
  return split_k_attention<0>(shape, o, q, k_pool, v_pool, k_new, v_new, new_slots, req_to_token, table_rows, stride,
                              seq_lens, batch, plan_dev, info, sm_scale, ws, RC_DECODE_STATIC_WORKSPACE_BYTES, stream,
                              false);
}

extern "C" rc_status rc_extend_attention_shared(const rc_shape* shape, void* o, const void* q, const void* k_pool,
                                                const void* v_pool, const int32_t* req_to_token, int32_t table_rows,
                                                int64_t stride, const int32_t* seq_lens, int32_t n_tokens,
                                                const int32_t* plan_dev, const rc_plan_info* info, float sm_scale,
                                                void* workspace, int64_t ws_bytes, void* stream) {
  return split_k_attention<1>(shape, o, q, const_cast<void*>(k_pool), const_cast<void*>(v_pool), nullptr, nullptr,
                              nullptr, req_to_token, table_rows, stride, seq_lens, n_tokens, plan_dev, info, sm_scale,
                              workspace, ws_bytes, stream);
}
