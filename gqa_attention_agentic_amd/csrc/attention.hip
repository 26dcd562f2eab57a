// Split-KV GQA flash attention for gfx950 (CDNA4), bf16 or fp32.
//
// Per work item (unit, KV head, M-tile, KV shard) a workgroup runs the
// FlashAttention tile loop of ADR-0060 GQA fused attention (TL;DR kernel
// and §3 per-tile op sequence) on the rows of its M-tile, 32 rows per wave:
//
//   S^T = K Q^T * scale      v_mfma_f32_32x32x16_bf16 (fp32: 32x32x2_f32)
//   mask                     only in tiles that cross the causal diagonal or
//                            the ragged end of the shard (§5.4 tile classes)
//   m' = max(m, rowmax S^T)  online softmax in fp32, log2 domain
//   P  = exp2(S^T - m'), l = l * 2^(m-m') + rowsum P
//   O^T = O^T * 2^(m-m') + V^T P^T
//
// Rows are (query token, g) pairs: the G query heads of a KV head and the
// tokens of every branch that shares the KV range are one M dimension
// (ADR-0060, §5.2; AHBM Agentic Runtime Architecture, §1.3 and §3.2), so a
// K/V tile read once into LDS serves all of them.
//
// Layout choices for CDNA4:
//  * S is computed transposed (keys x rows). In the 32x32 MFMA output a lane
//    then holds one row and 16 keys of it, so the row max / row sum are
//    in-lane plus a single exchange between the two half-waves, and the
//    rescale of O^T by 2^(m-m') is one scalar per lane.
//  * The S^T registers are already the B operand of V^T P^T (the contraction
//    index order is free as long as both operands agree), so P never leaves
//    registers.
//  * bf16 kernels stage K and V tiles into LDS with global->LDS DMA, rows
//    unpadded and XOR-swizzled per 16-byte chunk; V^T operands come from a
//    transposing LDS read. The fp32 kernels stage through registers (V is
//    transposed on the store, K rows padded).
//  * Wide kernels (MFMA-bound fan-out / prefill): bf16 256 rows (8 waves, a
//    4-stage ring of 64-key tiles consumed in pairs), fp32 128 rows (4
//    waves, double-buffered).
//  * Narrow kernels (KV-bandwidth-bound decode, <= 32 rows): every wave
//    streams its own 32-key tiles; the per-wave (m, l, O) states are merged
//    through LDS at the end, and tokens whose partials all come from narrow
//    items are combined inside the launch by the last item to finish.
//  * A row with exactly one live partial in total writes O / l and LSE
//    directly (ADR-0060, §0.5.4 N = 1); otherwise the unnormalised partial
//    (m, l, O) goes to the workspace for the combination (§4).
//  * Every workgroup runs the items of one bin (planned per resident
//    workgroup) back to back.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"

namespace gqa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T, int D, bool NARROW>
struct Cfg {
  static constexpr bool BF16 = std::is_same<T, uint16_t>::value;
  static constexpr int BN = NARROW ? kNarrowKeys : kWideKeys;   // keys per tile
  static constexpr int BM = NARROW ? kNarrowRows : kWideRows;   // rows per item
  static constexpr int LOADERS = NARROW ? 64 : 256;             // threads loading one tile
  static constexpr int VEC = 16 / (int)sizeof(T);               // elements per 16-byte chunk
  static constexpr int CHUNKS = BN * D / VEC;                   // chunks per tensor per tile
  static constexpr int CPT = CHUNKS / LOADERS;                  // chunks per thread per tensor
  static constexpr int KP = BF16 ? D + 8 : D + 1;               // K row pitch (elements)
  static constexpr int VP = BF16 ? BN + 8 : D + 4;              // V^T (bf16) / V (fp32) pitch
  static constexpr int K_ELEMS = BN * KP;
  static constexpr int V_ELEMS = BF16 ? D * VP : BN * VP;
  static constexpr int STAGE = ((K_ELEMS + V_ELEMS) * (int)sizeof(T) + 15) / 16 * 16;
  static constexpr int NSTAGE = NARROW ? 4 : 2;
  static constexpr int OB = D / 32;                             // O^T blocks per lane
  static constexpr int SB = BN / 32;                            // S^T blocks per tile
  static constexpr int QF = BF16 ? D / 16 : D / 2;              // Q fragments per lane
  static constexpr int MERGE = NARROW ? 4 * (OB * 16 * 64 + 2 * 64) * 4 : 0;
  static constexpr int LDS = (STAGE * NSTAGE > MERGE) ? STAGE * NSTAGE : MERGE;
  // Two workgroups per CU (8 waves, 2 per SIMD) when their LDS fits; the
  // register budget then is 256 per lane.
  static constexpr int WAVES_PER_SIMD = (!NARROW && 2 * LDS <= 160 * 1024) ? 2 : 1;
  static_assert(CHUNKS % LOADERS == 0, "tile does not split evenly over the loaders");
  static_assert(!BF16 || CPT == 2 || CPT % 4 == 0, "V transpose needs 2 or a multiple of 4 keys per thread");
  static_assert(LDS <= 160 * 1024, "LDS budget of a gfx950 CU exceeded");
};

template <class C>
struct Stage {
  uint4 k[C::CPT];
  uint4 v[C::CPT];
};

template <class C>
struct State {
  typename std::conditional<C::BF16, bf16x8_t, float>::type qf[C::QF];
  f32x16_t o[C::OB];
  float m;   // running max, log2 units
  float l;   // running sum
};

// Per-item K/V source: the shared prefix rows of one KV head (contiguous
// keys), or the branch's pages (one page-table lookup per key).
template <typename T>
struct KvSrc {
  const T* kb;            // shared: k_shared + (kv * n_shared + src) * D;  paged: k_pages + kv * ps * D
  const T* vb;
  const int32_t* table;   // paged: the branch's page-table row
  int64_t page_elems;     // paged: elements per page (H_kv * ps * D)
  int ps, shift;          // paged: page size and log2(page size) (-1 if not a power of two)
  bool paged;
};

template <typename T, int D, class U>
__device__ __forceinline__ KvSrc<T> kv_src(const AttnArgs& a, const U& u, int kv) {
  KvSrc<T> s;
  s.paged = u.kind != kShared;
  s.ps = a.page_size;
  s.shift = a.page_shift;
  if (!s.paged) {
    const int64_t base = ((int64_t)kv * a.n_shared + u.src) * D;
    s.kb = (const T*)a.k_shared + base;
    s.vb = (const T*)a.v_shared + base;
    s.table = nullptr;
    s.page_elems = 0;
  } else {
    const int64_t base = (int64_t)kv * a.page_size * D;
    s.kb = (const T*)a.k_pages + base;
    s.vb = (const T*)a.v_pages + base;
    s.table = a.page_table + (int64_t)u.src * a.max_pages;
    s.page_elems = (int64_t)a.H_kv * a.page_size * D;
  }
  return s;
}

// Element offset of unit-local key `key` in the source.
template <typename T, int D, bool PAGED>
__device__ __forceinline__ int64_t key_off(const KvSrc<T>& s, int key) {
  if (!PAGED) return (int64_t)key * D;
  int lp, slot;
  if (s.shift >= 0) {
    lp = key >> s.shift;
    slot = key & (s.ps - 1);
  } else {
    lp = key / s.ps;
    slot = key - lp * s.ps;
  }
  return (int64_t)s.table[lp] * s.page_elems + (int64_t)slot * D;
}

// Global -> registers for the KV tile whose first unit-local key is key0.
// Each thread loads CPT 16-byte chunks of K (consecutive lanes read
// consecutive chunks of a key row) and, for bf16, CPT consecutive keys of
// one 8-wide d slice of V (so it can write them transposed). Keys at or past
// key_end are not read (zero-filled) -- only checked when RAGGED.
template <class C, typename T, int D, bool PAGED, bool RAGGED>
__device__ __forceinline__ void load_tile_t(const KvSrc<T>& s, int key0, int key_end, int ltid,
                                            Stage<C>& st) {
  constexpr int CPR = D / C::VEC;   // chunks per key row
#pragma unroll
  for (int j = 0; j < C::CPT; ++j) {
    const int c = ltid + C::LOADERS * j;
    const int key = key0 + c / CPR;
    const int col = (c % CPR) * C::VEC;
    if (!RAGGED || key < key_end) {
      const int64_t off = key_off<T, D, PAGED>(s, key) + col;
      st.k[j] = *(const uint4*)(s.kb + off);
      if (!C::BF16) st.v[j] = *(const uint4*)(s.vb + off);
    } else {
      st.k[j] = make_uint4(0, 0, 0, 0);
      if (!C::BF16) st.v[j] = make_uint4(0, 0, 0, 0);
    }
  }
  if (C::BF16) {
    constexpr int KG = C::BN / C::CPT;
    const int kg = ltid % KG, oct = ltid / KG;
    const int k0 = key0 + kg * C::CPT;
    // CPT consecutive keys starting at a multiple of CPT never straddle a
    // page when the page size is a power-of-two multiple of CPT; otherwise
    // each key is looked up.
    const bool one_page = !PAGED || (s.shift >= 0 && s.ps >= C::CPT && (key0 & (C::CPT - 1)) == 0);
    const int64_t base = one_page ? key_off<T, D, PAGED>(s, k0) : 0;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int key = k0 + i;
      if (!RAGGED || key < key_end) {
        const int64_t off = (one_page ? base + (int64_t)i * D : key_off<T, D, PAGED>(s, key)) + oct * 8;
        st.v[i] = *(const uint4*)(s.vb + off);
      } else {
        st.v[i] = make_uint4(0, 0, 0, 0);
      }
    }
  }
}

template <class C, typename T, int D>
__device__ __forceinline__ void load_tile(const KvSrc<T>& s, int key0, int key_end, int ltid, Stage<C>& st) {
  const bool ragged = key0 + C::BN > key_end;
  if (s.paged) {
    if (ragged) load_tile_t<C, T, D, true, true>(s, key0, key_end, ltid, st);
    else load_tile_t<C, T, D, true, false>(s, key0, key_end, ltid, st);
  } else {
    if (ragged) load_tile_t<C, T, D, false, true>(s, key0, key_end, ltid, st);
    else load_tile_t<C, T, D, false, false>(s, key0, key_end, ltid, st);
  }
}

// Position of key k inside its 16-key chunk in the V^T LDS rows: bits 2 and
// 3 swapped, so that a lane's 8 P.V operand keys are 8 consecutive slots.
__device__ __forceinline__ int vt_slot(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <class C, typename T, int D>
__device__ __forceinline__ void store_tile(T* Ks, T* Vs, int ltid, const Stage<C>& st) {
  constexpr int CPR = D / C::VEC;
#pragma unroll
  for (int j = 0; j < C::CPT; ++j) {
    const int c = ltid + C::LOADERS * j;
    const int key = c / CPR;
    const int col = (c % CPR) * C::VEC;
    if (C::BF16) {
      *(uint4*)(Ks + key * C::KP + col) = st.k[j];
    } else {
      float* kd = (float*)Ks + key * C::KP + col;
      kd[0] = __uint_as_float(st.k[j].x);
      kd[1] = __uint_as_float(st.k[j].y);
      kd[2] = __uint_as_float(st.k[j].z);
      kd[3] = __uint_as_float(st.k[j].w);
      *(uint4*)((float*)Vs + key * C::VP + col) = st.v[j];
    }
  }
  if (C::BF16) {
    constexpr int KG = C::BN / C::CPT;
    const int kg = ltid % KG, oct = ltid / KG;
    uint16_t* vt = (uint16_t*)Vs;
#pragma unroll
    for (int di = 0; di < 8; ++di) {
      uint16_t* row = vt + (oct * 8 + di) * C::VP;
      const int sh = (di & 1) * 16;
#define GQA_HALF(i) ((((const uint32_t*)&st.v[i])[di >> 1] >> sh) & 0xffffu)
      if (C::CPT == 2) {
        const int k0 = kg * 2;
        const int slot = (k0 & ~15) | vt_slot(k0 & 15);
        *(uint32_t*)(row + slot) = GQA_HALF(0) | (GQA_HALF(1) << 16);
      } else {
#pragma unroll
        for (int run = 0; run < C::CPT / 4; ++run) {
          const int k0 = kg * C::CPT + run * 4;
          const int slot = (k0 & ~15) | vt_slot(k0 & 15);
          uint2 w;
          w.x = GQA_HALF(run * 4 + 0) | (GQA_HALF(run * 4 + 1) << 16);
          w.y = GQA_HALF(run * 4 + 2) | (GQA_HALF(run * 4 + 3) << 16);
          *(uint2*)(row + slot) = w;
        }
      }
#undef GQA_HALF
    }
  }
}

// One KV tile for one wave's 32 rows: S^T, mask, online softmax, O^T += V^T P^T.
// Scores stay unscaled until the exponent: p = exp2(s * c - m) with
// c = softmax_scale * log2(e) and the running max m kept in those units.
template <class C, typename T, int D, bool MASK>
__device__ __forceinline__ void compute_tile(const T* Ks, const T* Vs, State<C>& s, int kpos0,
                                             int n_valid, int causal, int row_pos, float c, int i,
                                             int h) {
  f32x16_t sacc[C::SB];
#pragma unroll
  for (int kb = 0; kb < C::SB; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
    if constexpr (C::BF16) {
      // Bound how many K operands the scheduler keeps in flight (register budget).
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8_t av = *(const bf16x8_t*)(Ks + (32 * kb + i) * C::KP + 16 * ks + 8 * h);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, s.qf[ks], sacc[kb], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < D / 2; ++ks) {
        const float av = ((const float*)Ks)[(32 * kb + i) * C::KP + 2 * ks + h];
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, s.qf[ks], sacc[kb], 0, 0, 0);
      }
    }
  }
  if (MASK) {
#pragma unroll
    for (int kb = 0; kb < C::SB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl = 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
        const bool vis = kl < n_valid && (!causal || kpos0 + kl <= row_pos);
        sacc[kb][r] = vis ? sacc[kb][r] : kNegInf;
      }
    }
  }
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < C::SB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sacc[kb][r], sacc[kb][r + 1]));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(s.m, mx * c);
  const float m_use = (m_new == kNegInf) ? 0.f : m_new;
  const float corr = exp2_fast(s.m - m_use);
  float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
  for (int kb = 0; kb < C::SB; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = exp2_fast(__builtin_fmaf(sacc[kb][r], c, -m_use));
      const float p1 = exp2_fast(__builtin_fmaf(sacc[kb][r + 1], c, -m_use));
      sacc[kb][r] = p0;
      sacc[kb][r + 1] = p1;
      rs0 += p0;
      rs1 += p1;
    }
  }
  float rs = rs0 + rs1;
  rs += __shfl_xor(rs, 32);
  s.l = s.l * corr + rs;
  s.m = m_new;
  // The running max rarely moves after the first tiles: skip the O rescale
  // when it moved for no row of the wave.
  if (__builtin_amdgcn_ballot_w64(corr != 1.f) != 0) {
#pragma unroll
    for (int db = 0; db < C::OB; ++db) s.o[db] *= corr;
  }

  if constexpr (C::BF16) {
#pragma unroll
    for (int kb = 0; kb < C::SB; ++kb) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        bf16x8_t pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sacc[kb][8 * cc + e];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < C::OB; ++db) {
          const bf16x8_t av =
              *(const bf16x8_t*)(Vs + (32 * db + i) * C::VP + (2 * kb + cc) * 16 + 8 * h);
          s.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb, s.o[db], 0, 0, 0);
        }
      }
    }
  } else {
#pragma unroll
    for (int kb = 0; kb < C::SB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
        for (int db = 0; db < C::OB; ++db) {
          const float av = ((const float*)Vs)[key * C::VP + 32 * db + i];
          s.o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, sacc[kb][r], s.o[db], 0, 0, 0);
        }
      }
    }
  }
}

// Tile dispatch: the mask is only built for tiles that cross the causal
// diagonal or the ragged end of the shard (ADR-0060, §5.4: all-past tiles
// carry no mask; all-future tiles were skipped by the caller).
template <class C, typename T, int D>
__device__ __forceinline__ void run_tile(const T* Ks, const T* Vs, State<C>& s, int key_pos0,
                                         int tk0, int key_end, int causal, int row_pos, int pmin,
                                         float c, int i, int h) {
  const int nvalid = min(C::BN, key_end - tk0);
  const int kpos0 = key_pos0 + tk0;
  const bool need_mask = (nvalid < C::BN) || (causal && kpos0 + C::BN - 1 > pmin);
  if (need_mask) compute_tile<C, T, D, true>(Ks, Vs, s, kpos0, nvalid, causal, row_pos, c, i, h);
  else compute_tile<C, T, D, false>(Ks, Vs, s, kpos0, nvalid, causal, row_pos, c, i, h);
}

// Per-lane row bookkeeping: row rloc of the item, i.e. the (token, g)
// pair number row_begin + rloc of its unit. The token record gives the
// position (for the causal mask) and whether the row's only partial is the
// result. One load, with no dependence on any other record.
struct Row {
  int tok, g, pos;
  bool ok;       // a valid row of the item
  bool direct;   // exactly one live partial: O / l and the LSE are written directly
};

__device__ __forceinline__ Row row_at(const AttnArgs& a, const WorkItem& it, int rloc) {
  Row w;
  w.ok = rloc < it.n_rows;
  const int r = it.row_begin + rloc;
  w.tok = it.tok_begin + r / a.G;
  w.g = r - (r / a.G) * a.G;
  w.pos = -1;
  w.direct = false;
  if (w.ok) {
    const TokRec tr = a.tok_rec[w.tok];
    w.pos = tr.pos;
    w.direct = tr.comb < 0;
  }
  return w;
}

template <class C, typename T, int D>
__device__ __forceinline__ void load_q(const AttnArgs& a, const Row& w, int kv, int h, State<C>& s) {
  const T* q = (const T*)a.q + ((int64_t)w.tok * a.H_q + kv * a.G + w.g) * D;
#pragma unroll
  for (int f = 0; f < C::QF; ++f) {
    if constexpr (C::BF16) {
      uint4 x = w.ok ? *(const uint4*)(q + 16 * f + 8 * h) : make_uint4(0, 0, 0, 0);
      s.qf[f] = __builtin_bit_cast(bf16x8_t, x);
    } else {
      s.qf[f] = w.ok ? ((const float*)q)[2 * f + h] : 0.f;
    }
  }
#pragma unroll
  for (int db = 0; db < C::OB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) s.o[db][r] = 0.f;
  s.m = kNegInf;
  s.l = 0.f;
}

// Where one lane's row goes: the output row itself when the row has exactly
// one live partial in total (written normalised, with its LSE), else this
// item's slot in the partial workspace.
struct RowDest {
  bool direct;
  int64_t row;   // direct: (token, head) index into o / lse; else the partial row
};

__device__ __forceinline__ RowDest row_dest(const AttnArgs& a, const WorkItem& it, const Row& w, int rloc) {
  RowDest d;
  d.direct = w.direct;
  d.row = w.direct ? (int64_t)w.tok * a.H_q + it.kv * a.G + w.g : it.part_row + rloc;
  return d;
}

// An 8-byte store at device scope: on gfx950 it is written through to the
// device's coherence point, so once the issuing thread's stores have
// completed (vmcnt 0) any CU of any XCD that acquires at device scope reads
// it -- no L2 write-back fence is needed for it.
__device__ __forceinline__ void store_device(void* p, float x, float y) {
  const uint64_t v = ((uint64_t)__float_as_uint(y) << 32) | __float_as_uint(x);
  __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Final or partial write of one lane's row for O^T blocks [db0, db1).
// COHERENT: the partial is written with device-scope stores (see
// combine_if_last).
template <class C, typename T, int D, bool COHERENT = false>
__device__ __forceinline__ void write_row_to(const AttnArgs& a, const RowDest& dst, bool ok, float m, float l,
                                             const f32x16_t* o, int db0, int db1, bool write_scalars, int h) {
  if (!ok) return;
  if (dst.direct) {
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    const int64_t orow = dst.row * D;
    for (int db = db0; db < db1; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * db + 8 * q4 + 4 * h;
        const float x0 = o[db - db0][4 * q4 + 0] * inv, x1 = o[db - db0][4 * q4 + 1] * inv;
        const float x2 = o[db - db0][4 * q4 + 2] * inv, x3 = o[db - db0][4 * q4 + 3] * inv;
        if constexpr (C::BF16) {
          uint2 pk;
          pk.x = pack_bf16x2(x0, x1);
          pk.y = pack_bf16x2(x2, x3);
          *(uint2*)((uint16_t*)a.o + orow + d0) = pk;
        } else {
          *(float4*)((float*)a.o + orow + d0) = make_float4(x0, x1, x2, x3);
        }
      }
    }
    if (write_scalars && h == 0) a.lse[dst.row] = (l > 0.f) ? (m + __log2f(l)) * kLn2 : kNegInf;
  } else {
    float* po = a.part_o + dst.row * D;
    for (int db = db0; db < db1; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * db + 8 * q4 + 4 * h;
        if (COHERENT) {
          store_device(po + d0, o[db - db0][4 * q4 + 0], o[db - db0][4 * q4 + 1]);
          store_device(po + d0 + 2, o[db - db0][4 * q4 + 2], o[db - db0][4 * q4 + 3]);
        } else {
          *(float4*)(po + d0) = make_float4(o[db - db0][4 * q4 + 0], o[db - db0][4 * q4 + 1],
                                            o[db - db0][4 * q4 + 2], o[db - db0][4 * q4 + 3]);
        }
      }
    }
    if (write_scalars && h == 0) {
      if (COHERENT) store_device(&a.part_ml[dst.row], m, l);
      else a.part_ml[dst.row] = make_float2(m, l);
    }
  }
}

// The same for the entry groups q0 .. q0 + NQ - 1 of O^T block db, given as
// float4s (entries 4 q .. 4 q + 3 of the block's accumulator).
template <typename T, int D, bool COHERENT, int NQ>
__device__ __forceinline__ void write_row_groups(const AttnArgs& a, const RowDest& dst, bool ok, float m, float l,
                                                 const float4 (&v)[NQ], int db, int q0, bool write_scalars, int h) {
  if (!ok) return;
  if (dst.direct) {
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    const int64_t orow = dst.row * D;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int d0 = 32 * db + 8 * (q0 + j) + 4 * h;
      if constexpr (std::is_same<T, uint16_t>::value) {
        uint2 pk;
        pk.x = pack_bf16x2(v[j].x * inv, v[j].y * inv);
        pk.y = pack_bf16x2(v[j].z * inv, v[j].w * inv);
        *(uint2*)((uint16_t*)a.o + orow + d0) = pk;
      } else {
        *(float4*)((float*)a.o + orow + d0) = make_float4(v[j].x * inv, v[j].y * inv, v[j].z * inv, v[j].w * inv);
      }
    }
    if (write_scalars && h == 0) a.lse[dst.row] = (l > 0.f) ? (m + __log2f(l)) * kLn2 : kNegInf;
  } else {
    float* po = a.part_o + dst.row * D;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int d0 = 32 * db + 8 * (q0 + j) + 4 * h;
      if (COHERENT) {
        store_device(po + d0, v[j].x, v[j].y);
        store_device(po + d0 + 2, v[j].z, v[j].w);
      } else {
        *(float4*)(po + d0) = v[j];
      }
    }
    if (write_scalars && h == 0) {
      if (COHERENT) store_device(&a.part_ml[dst.row], m, l);
      else a.part_ml[dst.row] = make_float2(m, l);
    }
  }
}

template <class C, typename T, int D>
__device__ __forceinline__ void write_row(const AttnArgs& a, const WorkItem& it, const Row& w, int rloc,
                                          float m, float l, const f32x16_t* o, int db0, int db1,
                                          bool write_scalars, int h) {
  if (!w.ok) return;
  write_row_to<C, T, D>(a, row_dest(a, it, w, rloc), true, m, l, o, db0, db1, write_scalars, h);
}

// ------------------------------------------------------- combination ----
// Log-sum-exp combination of the split-KV partials of an output row (tok,
// kv, g) (ADR-0060 GQA fused attention, §4: m = max m_i, weights
// 2^(m_i - m), one normalisation at the end). A row's partials are taken in
// a fixed order -- prefix shards, then suffix shards -- so the result does
// not depend on which workgroup combines it. Rows with a single partial
// were written by their item directly.

// Workspace row of partial q of row (g, kv) of a token with combination
// record c: the prefix unit's shards first, then the suffix unit's.
__device__ __forceinline__ int64_t part_of(const CombTok& c, int kv, int g, int q) {
  const bool pre = q < c.live[0];
  const int64_t p = pre ? c.p[0] : c.p[1];
  const int live = pre ? c.live[0] : c.live[1], stride = pre ? c.stride[0] : c.stride[1];
  const int sh = pre ? q : q - c.live[0];
  return p + ((int64_t)kv * live + sh) * stride + g;
}

// (M, L, O) <- the combination of (M, L, O) and (M2, L2, O2), in that order.
__device__ __forceinline__ void join_state(float& M, float& L, float4& O, float M2, float L2, const float4& O2) {
  const float Mn = fmaxf(M, M2);
  const float Mu = (Mn == kNegInf) ? 0.f : Mn;
  const float sa = exp2_fast(M - Mu), sb = exp2_fast(M2 - Mu);
  L = L * sa + L2 * sb;
  O.x = O.x * sa + O2.x * sb;
  O.y = O.y * sa + O2.y * sb;
  O.z = O.z * sa + O2.z * sb;
  O.w = O.w * sa + O2.w * sb;
  M = Mn;
}

// Folds partials [q_begin, q_end) of row (g, kv) into (M, L, O) for the d
// values d0 .. d0 + 3, one after another; U partial loads are issued before
// they are consumed.
template <int D, int U>
__device__ __forceinline__ void fold_parts(const AttnArgs& a, const CombTok& c, int kv, int g, int q_begin, int q_end,
                                           int d0, float& M, float& L, float4& O) {
  for (int q0 = q_begin; q0 < q_end; q0 += U) {
    float2 ml[U];
    float4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int q = q0 + k;
      if (q < q_end) {
        const int64_t p = part_of(c, kv, g, q);
        ml[k] = a.part_ml[p];
        v[k] = *(const float4*)(a.part_o + p * D + d0);
      } else {
        ml[k] = make_float2(kNegInf, 0.f);
        v[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) join_state(M, L, O, ml[k].x, ml[k].y, v[k]);
  }
}

// O / L in the storage dtype (round to nearest even) and, from the thread
// holding d0 = 0, LSE = ln L + M ln 2.
template <typename T, int D>
__device__ __forceinline__ void write_combined(const AttnArgs& a, int tok, int kv, int g, int d0, float M, float L,
                                               const float4& O) {
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  const int64_t orow = ((int64_t)tok * a.H_q + kv * a.G + g);
  if constexpr (std::is_same<T, uint16_t>::value) {
    uint2 pk;
    pk.x = pack_bf16x2(O.x * inv, O.y * inv);
    pk.y = pack_bf16x2(O.z * inv, O.w * inv);
    *(uint2*)((uint16_t*)a.o + orow * D + d0) = pk;
  } else {
    *(float4*)((float*)a.o + orow * D + d0) = make_float4(O.x * inv, O.y * inv, O.z * inv, O.w * inv);
  }
  if (d0 == 0) a.lse[orow] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : kNegInf;
}

// Folds the partials of row (tok, g) of KV head kv, whose combination
// record is c, and writes its O and LSE. RL = D / 2 lanes take the row, this
// one being number j of them (lane0: the first of them in the wave): lanes 2y
// and 2y + 1 own the row's d values 4y .. 4y + 3, and each folds every other
// partial. The lanes first take one partial's (m, l) each, so that the row's
// maximum M, and each partial's weight 2^(m_i - M), are formed once,
// lane-parallel; the weights reach the O lanes by a lane exchange. The sum
// runs in a fixed order.
template <typename T, int D>
__device__ __forceinline__ void fold_row(const AttnArgs& a, const CombTok& c, int kv, int tok, int g, int j,
                                         int lane0) {
  constexpr int RL = D / 2;
  const int n = c.live[0] + c.live[1];
  const int half = j & 1, d0 = (j >> 1) * 4;
  constexpr int U = 8;                      // partial loads in flight per lane
  // The row's first RL partials' (m, l), one per lane, and this lane's
  // first U partials' O values go out together: the O loads do not wait
  // for the weights.
  float2 ml0 = make_float2(kNegInf, 0.f);
  if (j < n) ml0 = a.part_ml[part_of(c, kv, g, j)];
  const int cnt0 = min(RL, n);
  float4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int kk = 2 * u + half;
    v[u] = kk < cnt0 ? *(const float4*)(a.part_o + part_of(c, kv, g, kk) * D + d0)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float M = ml0.x;
  for (int c0 = RL; c0 < n; c0 += RL)
    if (c0 + j < n) M = fmaxf(M, a.part_ml[part_of(c, kv, g, c0 + j)].x);
#pragma unroll
  for (int sh = 1; sh < RL; sh <<= 1) M = fmaxf(M, __shfl_xor(M, sh));
  const float Mu = (M == kNegInf) ? 0.f : M;
  float L = 0.f;
  float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = 0; c0 < n; c0 += RL) {
    float2 ml = ml0;
    if (c0 > 0) ml = (c0 + j < n) ? a.part_ml[part_of(c, kv, g, c0 + j)] : make_float2(kNegInf, 0.f);
    const float wq = exp2_fast(ml.x - Mu);  // 0 for an empty partial (m = -inf)
    L += wq * ml.y;
    const int cnt = min(RL, n - c0);
    for (int t0 = 0; t0 < cnt; t0 += 2 * U) {
      if (c0 > 0 || t0 > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int kk = t0 + 2 * u + half;
          v[u] = kk < cnt ? *(const float4*)(a.part_o + part_of(c, kv, g, c0 + kk) * D + d0)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = t0 + 2 * u + half;
        const float wu = __shfl(wq, lane0 + min(kk, cnt - 1)) * (kk < cnt ? 1.f : 0.f);
        O.x += wu * v[u].x;
        O.y += wu * v[u].y;
        O.z += wu * v[u].z;
        O.w += wu * v[u].w;
      }
    }
  }
#pragma unroll
  for (int sh = 1; sh < RL; sh <<= 1) L += __shfl_xor(L, sh);
  O.x += __shfl_xor(O.x, 1);
  O.y += __shfl_xor(O.y, 1);
  O.z += __shfl_xor(O.z, 1);
  O.w += __shfl_xor(O.w, 1);
  if (half == 0) write_combined<T, D>(a, tok, kv, g, d0, M, L, O);
}

// s_waitcnt immediate: vmcnt(vm), expcnt(7), lgkmcnt(0).
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | (7 << 4) | (0 << 8) | ((vm >> 4) << 14); }

// A load of plan data (written before the launch and constant during it) at
// a wave-uniform address, made through the constant address space so that
// it is a scalar load: scalar loads are counted apart from vector memory
// operations, so waiting for one never waits for K/V loads in flight.
template <typename T>
__device__ __forceinline__ T plan_load(const T* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return *(const __attribute__((address_space(4))) T*)p;
#else
  return *p;
#endif
}

// In-launch combination (narrow kernels). Tokens whose partials all come
// from narrow items (decode-like rows: a few rows over a long KV range cut
// into many shards) are combined by the last of their items to finish,
// which spares them the separate merge launch; the MFMA-bound items leave
// theirs to lse_merge, since a combining workgroup would stall its CU.
//  * At the item's start, while its K/V stream is in flight, wave 0 copies
//    the combination records of the item's tokens into LDS (a unit goes to
//    the narrow kernel only when all its rows fit one M-tile, so an item
//    has at most BM rows and tokens).
//  * After its rows are written, each such token's counter (one per KV
//    head, in the token's counter slot, a 128-byte line apart from every
//    other counter so that the items of different KV heads and tokens do
//    not queue their atomics on one line) is incremented; the item that
//    brings it to the planned number of arrivals combines the token's rows. The XCDs' L2 caches are not
//    coherent with each other, so every other item's partials must reach
//    device scope before its increment, and the winner acquires at device
//    scope after its own. Two ways:
//      - partials in ordinary stores, then a device-scope release fence
//        (write-back of the L2's dirty lines) before the increment;
//      - partials in device-scope stores (a.coherent_parts), which need
//        only to have completed before the increment. Used when every
//        workgroup runs a single item: all of them then finish at once,
//        and hundreds of simultaneous L2 write-backs queue up (measured on
//        MI355X: ~4.6 us from stores done to arrival at the 8k decode's 256
//        items); with several items per workgroup the arrivals are spread
//        out and ordinary stores plus the fence are cheaper.
//    The winner resets the counter after its combination, so all counters
//    are zero again when the launch ends. Work per workgroup is bounded and
//    no thread waits on another workgroup.
//  * The fold of a row (fold_row) takes D / 2 lanes: two per group of four
//    d values, each summing every other partial, joined by a lane exchange
//    at the end. Its cost is the bytes of the row's partials passing
//    through one CU's vector-memory path.
template <int BM>
struct CombLds {
  CombTok rec[BM];   // per token of the item (need = 0: combined elsewhere, or one partial)
  int won[BM];
  int kv, tok0, ntok;
};

template <int BM>
__device__ __forceinline__ void combine_prepare(const AttnArgs& a, const WorkItem& it, int wave, int lane,
                                                CombLds<BM>* cl) {
  if (wave != 0) return;
  // The item is wave-uniform; say so, so that the loads below are scalar.
  const int tok0 = __builtin_amdgcn_readfirstlane(it.tok_begin + it.row_begin / a.G);
  const int ntok = __builtin_amdgcn_readfirstlane(
      (it.n_rows > 0) ? it.tok_begin + (it.row_begin + it.n_rows - 1) / a.G - tok0 + 1 : 0);
  for (int k = 0; k < ntok; ++k) {
    const int ci = plan_load(&a.tok_rec[tok0 + k].comb);
    CombTok c;
    if (ci >= 0) {
      const CombTok* src = a.combs + ci;   // field by field: an aggregate copy would not be scalar
      c.p[0] = plan_load(&src->p[0]);
      c.p[1] = plan_load(&src->p[1]);
      c.live[0] = plan_load(&src->live[0]);
      c.live[1] = plan_load(&src->live[1]);
      c.stride[0] = plan_load(&src->stride[0]);
      c.stride[1] = plan_load(&src->stride[1]);
      c.need = plan_load(&src->need);
      c.slot = plan_load(&src->slot);
    } else {
      c.p[0] = c.p[1] = 0;
      c.live[0] = c.live[1] = 0;
      c.stride[0] = c.stride[1] = 0;
      c.need = 0;
      c.slot = -1;
    }
    if (lane == 0) cl->rec[k] = c;
  }
  if (lane == 0) {
    cl->kv = it.kv;
    cl->tok0 = tok0;
    cl->ntok = ntok;
  }
}

template <typename T, int D, int NT, int BM>
__device__ __forceinline__ void combine_if_last(const AttnArgs& a, int tid, CombLds<BM>* cl) {
  // vmcnt counts stores too: every wave's partial stores are complete at
  // the barrier, so the release below covers them.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  __syncthreads();
  const int kv = cl->kv, tok0 = cl->tok0, ntok = cl->ntok;
  for (int k = tid; k < ntok; k += NT) {
    const int need = cl->rec[k].need;
    int w = 0;
    if (need > 0) {
      int* c = a.counters + ((int64_t)cl->rec[k].slot * a.H_kv + kv) * kCounterStride;
      if (!a.coherent_parts) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      if (atomicAdd(c, 1) == need - 1) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        w = 1;
      }
    }
    cl->won[k] = w;
  }
  // Whether any of the item's tokens is combined here, from the flags in
  // LDS (a workgroup OR-reduction would compile to a library call, whose
  // register saves cost the K/V stream loop registers).
  __syncthreads();
  int any = 0;
  for (int k = 0; k < ntok; ++k) any |= cl->won[k];
  if (!any) return;
  const int G = a.G;
  constexpr int RL = D / 2;   // lanes per row: two per group of four d values
  for (int x = tid; x < ntok * G * RL; x += NT) {
    const int rr = x / RL, j = x - rr * RL;   // row, lane within the row
    const int k = rr / G;
    if (!cl->won[k]) continue;                // the same for every lane of the row
    int lane = tid & 63;
    // Opaque, so that nothing derived from the lane index (the exchange
    // addresses of the fold) is hoisted out of the item loop and kept live
    // through the K/V stream.
    asm volatile("" : "+v"(lane));
    fold_row<T, D>(a, cl->rec[k], kv, tok0 + k, rr - k * G, j, lane - j);
  }
  int t = tid;
  asm volatile("" : "+v"(t));   // no LDS address of this loop is computed at the kernel's start and kept
  for (int k = t; k < ntok; k += NT)
    if (cl->won[k]) atomicExch(a.counters + ((int64_t)cl->rec[k].slot * a.H_kv + kv) * kCounterStride, 0);
}

// Smallest / largest valid row position of the wave.
__device__ __forceinline__ void wave_pos_range(const Row& w, int* pmin, int* pmax) {
  int lo = w.ok ? w.pos : 0x7fffffff, hi = w.ok ? w.pos : -1;
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) {
    lo = min(lo, __shfl_xor(lo, x));
    hi = max(hi, __shfl_xor(hi, x));
  }
  *pmin = __builtin_amdgcn_readfirstlane(lo);   // wave-uniform: keep in SGPRs
  *pmax = __builtin_amdgcn_readfirstlane(hi);
}

// ---------------------------------------------------------------- wide ----
template <typename T, int D>
__global__ void __launch_bounds__(256, (Cfg<T, D, false>::WAVES_PER_SIMD))
attn_wide(AttnArgs a) {
  using C = Cfg<T, D, false>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, i = lane & 31, h = lane >> 5;
  const int bin_end = a.bins[blockIdx.x + 1];
  State<C> s;   // carried from one item to the next along a chain
  for (int idx = a.bins[blockIdx.x]; idx < bin_end; ++idx) {
    // The previous item's last tile loop iteration ended with a barrier after
    // all LDS reads, so its stages may be refilled at once.
    const WorkItem it = a.items[idx];
    const int rloc = wave * 32 + i;
    const Row w = row_at(a, it, rloc);
    if (!(it.chain & kChainContinues)) load_q<C, T, D>(a, w, it.kv, h, s);
    int pmin, pmax;
    wave_pos_range(w, &pmin, &pmax);
    const bool wave_rows = wave * 32 < it.n_rows;
    const KvSrc<T> src = kv_src<T, D>(a, it, it.kv);

    const int nt = (it.key_end - it.key_begin + C::BN - 1) / C::BN;
    Stage<C> st;
    load_tile<C, T, D>(src, it.key_begin, it.key_end, tid, st);
    store_tile<C, T, D>((T*)smem, (T*)(smem + C::K_ELEMS * sizeof(T)), tid, st);
    __syncthreads();
    for (int j = 0; j < nt; ++j) {
      const bool more = j + 1 < nt;
      if (more) load_tile<C, T, D>(src, it.key_begin + (j + 1) * C::BN, it.key_end, tid, st);
      const int tk0 = it.key_begin + j * C::BN;       // unit-local first key of the tile
      const bool future = a.causal && (it.key_pos0 + tk0 > pmax);
      if (wave_rows && !future) {
        char* stg = smem + (j & 1) * C::STAGE;
        run_tile<C, T, D>((const T*)stg, (const T*)(stg + C::K_ELEMS * sizeof(T)), s, it.key_pos0, tk0, it.key_end,
                          a.causal, w.pos, pmin, a.scale_log2, i, h);
      }
      if (more) {
        char* stg = smem + ((j + 1) & 1) * C::STAGE;
        store_tile<C, T, D>((T*)stg, (T*)(stg + C::K_ELEMS * sizeof(T)), tid, st);
      }
      __syncthreads();
    }
    if (!(it.chain & kChainContinued)) write_row<C, T, D>(a, it, w, rloc, s.m, s.l, s.o, 0, C::OB, true, h);
  }
}

// ------------------------------------------------------ wide, bf16, DMA ----
// The MFMA-bound kernel for bf16: 8 waves (256 rows, 32 per wave, 2 waves
// per SIMD) share a 4-stage ring of 64-key K/V tiles in LDS that global->LDS
// DMA (global_load_lds_dwordx4) fills two tiles ahead of the compute, with
// no register staging. LDS rows are unpadded and XOR-swizzled per 16-byte
// chunk (swz_k / swz_v below) so that both operand reads are free of bank
// conflicts. The transposing LDS read turns V's [key][d] rows into the
// k-contiguous operand of O^T += V^T P^T without any transpose on the store
// side.
template <int D>
struct DmaCfg {
  static constexpr bool BF16 = true;
  static constexpr int WAVES = 8;
  static constexpr int THREADS = 64 * WAVES;        // launch size (every launch and occupancy query uses it)
  static constexpr int BM = 32 * WAVES;             // rows per item
  static constexpr int BN = 64;                     // keys per tile
  static constexpr int ROW = D * 2;                 // bytes per key row
  static constexpr int TB = BN * ROW;               // bytes per tensor per tile
  static constexpr int NINST = TB / 1024;           // 1 KB wave-instructions per tensor per tile
  static constexpr int PER_WAVE = NINST / WAVES;    // per tensor per wave
  static constexpr int VM_PER_TILE = 2 * PER_WAVE;  // DMA instructions per thread per tile
  static constexpr int OB = D / 32, QF = D / 16, SB = BN / 32;
  static_assert(NINST % WAVES == 0, "tile must split evenly over the waves");
  static_assert(BM == kWideRowsBf16, "planner and kernel disagree on the M-tile");
};

// The DMA below is issued as inline assembly, so the compiler neither counts
// it nor inserts waits for it (its own tracking of LDS DMA cannot tell ring
// stages apart and would make every LDS read wait for all DMA in flight).
// Every consumer waits explicitly with wait_dma<VM>(): at most VM of this
// thread's vector-memory operations still outstanding (they complete in
// order) and all its LDS operations done. Both carry a memory clobber, so
// the compiler moves no LDS access across them.
template <int VM>
__device__ __forceinline__ void wait_dma() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(VM));
  asm volatile("" ::: "memory");
}

// 16 bytes per lane from gptr into LDS: lane l writes lds_base + 16 l
// (lds_base wave-uniform, passed in M0; one wait state between the write of
// M0 and the load).
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gptr), "{m0}"(m0) : "memory");
}

// Workgroup barrier that is also a compiler barrier for memory and for the
// instruction scheduler.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// LDS byte address of a __shared__ object (or of an LDS pointer).
__device__ __forceinline__ uint32_t lds_u32(const char* p) {
  return (uint32_t)(uintptr_t)(const lds_char*)p;
}
__device__ __forceinline__ uint32_t lds_u32(const lds_char* p) { return (uint32_t)(uintptr_t)p; }

// LDS swizzle of a K or V tile row (one key, ROW bytes = ROW/16 chunks of 16
// bytes): logical chunk c of key k sits at physical chunk c ^ swz(k). The
// LDS serves 16 lanes of a 16-byte read (or 32 lanes of an 8-byte read) per
// cycle across 64 four-byte banks, i.e. 16 chunk slots, and a key row of
// d = 128 (256 bytes) covers all 16 slots, so:
//  * K operand (ds_read_b128): the 16 lanes of a cycle read one logical
//    chunk of 16 consecutive keys; XOR with key & 15 spreads them over all
//    16 slots (d = 64: rows alternate slot halves, XOR with bits 1..3).
//  * V operand (ds_read_b64_tr_b16): the 32 lanes of a cycle read 4
//    consecutive keys x 4 logical chunks; XOR with 4 (key & 3) moves each
//    key to its own group of 4 slots (d = 64: 4 ((key >> 1) & 1)).
template <int ROW>
__device__ __forceinline__ int swz_k(int key) {
  static_assert(ROW == 256 || ROW == 128, "swizzles are laid out for d = 128 and d = 64");
  return ROW == 256 ? (key & 15) : ((key >> 1) & 7);
}
template <int ROW>
__device__ __forceinline__ int swz_v(int key) {
  return ROW == 256 ? 4 * (key & 3) : 4 * ((key >> 1) & 1);
}

template <class C>
struct DmaLane {
  // per-lane constants of the DMA (global side) and of the operand reads (LDS side)
  int key_rel[C::PER_WAVE];   // tile-relative key of this lane's chunk in instruction q
  int colK[C::PER_WAVE];      // element offset inside the key row (logical chunk * 8)
  int colV[C::PER_WAVE];
  int kaddr[C::QF];           // byte offset of the K operand chunk for ks (key block kb adds kb * 32 rows)
  int vaddr[C::OB];           // byte offset of the V tr16 read for db (16-key chunk kc adds 16 kc rows)
};

template <class C>
__device__ __forceinline__ DmaLane<C> dma_lane(int wave, int lane) {
  DmaLane<C> L;
#pragma unroll
  for (int q = 0; q < C::PER_WAVE; ++q) {
    const int byte = (wave * C::PER_WAVE + q) * 1024 + 16 * lane;
    const int kr = byte / C::ROW;
    const int pc = (byte % C::ROW) / 16;
    L.key_rel[q] = kr;
    L.colK[q] = (pc ^ swz_k<C::ROW>(kr)) * 8;
    L.colV[q] = (pc ^ swz_v<C::ROW>(kr)) * 8;
  }
  const int i = lane & 31, h = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < C::QF; ++ks) L.kaddr[ks] = i * C::ROW + 16 * ((2 * ks + h) ^ swz_k<C::ROW>(i));
  // V^T fragment through ds_read_b64_tr_b16: in 16-lane group g, lane j
  // supplies 4 elements of key 4 (g >> 1) + (j >> 2), d = 32 db + 16 (g & 1)
  // + 4 (j & 3); the transpose hands lane j of the group d = ... + j for 4
  // consecutive keys.
  const int g = lane >> 4, j = lane & 15, half = g & 1, hh = g >> 1;
  const int key0 = 4 * hh + (j >> 2);
#pragma unroll
  for (int db = 0; db < C::OB; ++db)
    L.vaddr[db] = key0 * C::ROW + 16 * ((4 * db + 2 * half + ((j >> 1) & 1)) ^ swz_v<C::ROW>(key0)) + 8 * (j & 1);
  return L;
}

// Issue the DMA of tile `t` (unit-local first key key0) into one ring stage.
// Keys past key_end are clamped to the last valid key (finite data, masked
// later). Paged sources with power-of-two pages of >= 16 tokens look up the
// ids of the at most five pages the tile touches, not one id per key; those
// lookups are loads the DMA addresses wait for. With PRE, the ids of pages
// lp0 .. lp0 + 4 (clamped to the unit's last page) come in `pre` instead,
// read ahead by the caller (page_ids_ahead).
template <class C, int D, bool PAGED, bool SCALAR_PAGES, int WHICH, bool PRE = false>
__device__ __forceinline__ void dma_tile(const KvSrc<uint16_t>& src, const DmaLane<C>& L, int wave, int key0,
                                         int key_end, uint32_t Kst, uint32_t Vst, const int* pre = nullptr) {
  int pg[5] = {0, 0, 0, 0, 0};
  int lp0 = 0;
  if (PAGED && SCALAR_PAGES) {
    lp0 = key0 >> src.shift;
    const int lp_last = (key_end - 1) >> src.shift;
#pragma unroll
    for (int e = 0; e < 5; ++e) pg[e] = PRE ? pre[e] : src.table[min(lp0 + e, lp_last)];
  }
#pragma unroll
  for (int q = 0; q < C::PER_WAVE; ++q) {
    const int k = min(key0 + L.key_rel[q], key_end - 1);
    int64_t off;
    if (!PAGED) {
      off = (int64_t)k * D;
    } else if (SCALAR_PAGES) {
      const int e = (k >> src.shift) - lp0;
      int page = pg[0];
      page = (e == 1) ? pg[1] : page;
      page = (e == 2) ? pg[2] : page;
      page = (e == 3) ? pg[3] : page;
      page = (e == 4) ? pg[4] : page;
      off = (int64_t)page * src.page_elems + (int64_t)(k & (src.ps - 1)) * D;
    } else {
      off = key_off<uint16_t, D, true>(src, k);
    }
    const int n = wave * C::PER_WAVE + q;
    if (WHICH & 1) dma16(src.kb + off + L.colK[q], Kst + n * 1024);
    if (WHICH & 2) dma16(src.vb + off + L.colV[q], Vst + n * 1024);
  }
}

// The page ids a tile starting at key0 needs (paged source, power-of-two
// pages of >= 16 tokens), as a vector load to be consumed one loop step
// later: lane e < 5 gets the id of logical page (key0 >> shift) + e, clamped
// to the unit's last page; lanes past 4 repeat lane 4's load. Issued right
// behind a tile's DMA, it lands with that tile, so the next DMA issue waits
// on no page-table round trip.
__device__ __forceinline__ int page_ids_ahead(const KvSrc<uint16_t>& src, int key0, int key_end, int lane) {
  const int lp0 = key0 >> src.shift, lp_last = (key_end - 1) >> src.shift;
  return src.table[min(lp0 + min(lane, 4), lp_last)];
}

template <class C, int D, int WHICH = 3, typename P>
__device__ __forceinline__ void dma_tile_any(const KvSrc<uint16_t>& src, const DmaLane<C>& L, int wave, int key0,
                                             int key_end, P* Kp, P* Vp) {
  const uint32_t Kst = lds_u32(Kp), Vst = lds_u32(Vp);
  if (!src.paged) dma_tile<C, D, false, false, WHICH>(src, L, wave, key0, key_end, Kst, Vst);
  else if (src.shift >= 4) dma_tile<C, D, true, true, WHICH>(src, L, wave, key0, key_end, Kst, Vst);
  else dma_tile<C, D, true, false, WHICH>(src, L, wave, key0, key_end, Kst, Vst);
}

// Scores of one tile for one wave, then the online softmax with a lazy
// rescale: the running max only moves (and O, l are rescaled) when some row
// of the wave sees a score more than 2^8 above it; otherwise p = 2^(s*c - m)
// stays below 256, which bf16 P and fp32 O, l hold exactly as well as
// smaller values. The result is the same softmax; only the reference point
// of the exponent differs between rescales. The P.V products are software
// pipelined in 16-key chunks: the exponentials and the V^T operand reads of
// chunk n + 1 are issued between chunk n's MFMAs (scheduling fences keep
// the compiler from regrouping them), so the softmax VALU work runs in the
// matrix core's shadow.
// Lane bases of the wide kernel's operand reads in its contiguous ring.
template <class C>
struct RingLane {
  uint32_t kaddr[C::QF];   // LDS address of the K operand chunk for ks in stage 0 (this lane)
  uint32_t vaddr[C::OB];   // LDS address of the V tr16 read for db in stage 0 (this lane)
};

template <class C, int D, bool MASK, int STAGE = -1, class LA = DmaLane<C>>
__device__ __forceinline__ void dma_compute(uint32_t kst, uint32_t vst, const LA& L,
                                            State<C>& s, int kpos0, int n_valid, int causal,
                                            int row_pos, float c, int i, int h) {
  constexpr float kTau = 8.f;
  typedef __attribute__((address_space(3))) const bf16x8_t* lds_bf16x8;
  typedef __attribute__((address_space(3))) v4i16_t* lds_v4i16;
  uint32_t kbs[C::QF], vbs[C::OB];
  if constexpr (STAGE >= 0) {
    // Lane bases fixed for the whole launch; the stage is an immediate offset.
#pragma unroll
    for (int q = 0; q < C::QF; ++q) kbs[q] = L.kaddr[q] + STAGE * C::TB;
#pragma unroll
    for (int q = 0; q < C::OB; ++q) vbs[q] = L.vaddr[q] + STAGE * C::TB;
  } else {
    // Per-call opaque bases: every operand address below is base + immediate.
#pragma unroll
    for (int q = 0; q < C::QF; ++q) {
      kbs[q] = kst + L.kaddr[q];
      asm volatile("" : "+v"(kbs[q]));
    }
#pragma unroll
    for (int q = 0; q < C::OB; ++q) {
      vbs[q] = vst + L.vaddr[q];
      asm volatile("" : "+v"(vbs[q]));
    }
  }
  f32x16_t sacc[C::SB];
#pragma unroll
  for (int kb = 0; kb < C::SB; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8_t av = *(lds_bf16x8)(uintptr_t)(kbs[ks] + kb * 32 * C::ROW);
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, s.qf[ks], sacc[kb], 0, 0, 0);
    }
  }
  if (MASK) {
    // Key kl = (compile-time part) + 4h of the tile is visible iff kl <
    // n_valid and (causal) kpos0 + kl <= row_pos: one compare per score of
    // the constant part against a per-lane limit.
    const int lim = min(n_valid, causal ? row_pos - kpos0 + 1 : n_valid) - 4 * h;
#pragma unroll
    for (int kb = 0; kb < C::SB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sacc[kb][r] = (32 * kb + 8 * (r >> 2) + (r & 3) < lim) ? sacc[kb][r] : kNegInf;
  }
  // A chain of two-input maxima, which the compiler fuses pairwise into
  // v_max3_f32: one instruction per two scores (16 per tile, against 24
  // when each pair is reduced first).
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < C::SB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, sacc[kb][r]), sacc[kb][r + 1]);
  // Lane-local max over its half of the row's keys: the rescale decision
  // needs no exchange (the ballot spans the wave); only an actual rescale
  // combines the two halves' maxima, so both keep the same m.
  mx *= c;
  if (__builtin_amdgcn_ballot_w64(mx > s.m + kTau) != 0) {
    const float m_new = __builtin_fmaxf(s.m, __builtin_fmaxf(mx, __shfl_xor(mx, 32)));
    const float corr = (m_new == kNegInf) ? 1.f : exp2_fast(s.m - m_new);
    s.l *= corr;
#pragma unroll
    for (int db = 0; db < C::OB; ++db) s.o[db] *= corr;
    s.m = m_new;
  }
  const float neg_m = (s.m == kNegInf) ? 0.f : -s.m;
  // Chunk n = 16 keys of the tile (S^T block n / 2, accumulator entries
  // 8 (n % 2) .. +7 of this lane).
  constexpr int NCH = 2 * C::SB;
  float r0 = 0.f, r1 = 0.f;
  bf16x8_t pb[2];
  auto make_p = [&](int n, bf16x8_t& out) {
    const int kb = n >> 1, r = 8 * (n & 1);
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float p0 = exp2_fast(__builtin_fmaf(sacc[kb][r + e], c, neg_m));
      const float p1 = exp2_fast(__builtin_fmaf(sacc[kb][r + e + 1], c, neg_m));
      r0 += p0;
      r1 += p1;
      out[e] = (__bf16)p0;
      out[e + 1] = (__bf16)p1;
    }
  };
  auto v_frag = [&](int n, int db) -> bf16x8_t {
    const uint32_t va = vbs[db] + (16 * n) * C::ROW;
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16)(uintptr_t)va);
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16)(uintptr_t)(va + 8 * C::ROW));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  bf16x8_t vf[C::OB];
  make_p(0, pb[0]);
#pragma unroll
  for (int db = 0; db < C::OB; ++db) vf[db] = v_frag(0, db);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int n = 0; n < NCH; ++n) {
    const int cur = n & 1;
#pragma unroll
    for (int db = 0; db < C::OB; ++db) {
      s.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db], pb[cur], s.o[db], 0, 0, 0);
      if (n + 1 < NCH) vf[db] = v_frag(n + 1, db);
      if (db == 1 && n + 1 < NCH) make_p(n + 1, pb[cur ^ 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  s.l += r0 + r1;   // sum over this lane's keys; the two halves are added once, at the end
}

template <class C, int D>
__device__ __forceinline__ void dma_step(uint32_t kst, uint32_t vst, const DmaLane<C>& L, State<C>& s,
                                         int key_pos0, int tk0, int key_end, int causal, int row_pos,
                                         int pmin, int pmax, bool active, float c, int i, int h) {
  const int kpos0 = key_pos0 + tk0;
  if (!active || (causal && kpos0 > pmax)) return;   // no rows, or the tile is all-future for the wave
  const int nvalid = min(C::BN, key_end - tk0);
  const bool need_mask = (nvalid < C::BN) || (causal && kpos0 + C::BN - 1 > pmin);
  if (need_mask) dma_compute<C, D, true>(kst, vst, L, s, kpos0, nvalid, causal, row_pos, c, i, h);
  else dma_compute<C, D, false>(kst, vst, L, s, kpos0, nvalid, causal, row_pos, c, i, h);
}

// The same for a tile in stage STAGE of the wide kernel's contiguous ring.
template <class C, int D, int STAGE>
__device__ __forceinline__ void dma_step_ring(const RingLane<C>& R, State<C>& s, int key_pos0, int tk0, int key_end,
                                              int causal, int row_pos, int pmin, int pmax, bool active, float c,
                                              int i, int h) {
  const int kpos0 = key_pos0 + tk0;
  if (!active || (causal && kpos0 > pmax)) return;
  const int nvalid = min(C::BN, key_end - tk0);
  const bool need_mask = (nvalid < C::BN) || (causal && kpos0 + C::BN - 1 > pmin);
  if (need_mask) dma_compute<C, D, true, STAGE, RingLane<C>>(0, 0, R, s, kpos0, nvalid, causal, row_pos, c, i, h);
  else dma_compute<C, D, false, STAGE, RingLane<C>>(0, 0, R, s, kpos0, nvalid, causal, row_pos, c, i, h);
}


// Four ring stages consumed two tiles per barrier: after the barrier of pair
// p (tiles 2p, 2p+1) the DMA of pair p+1 is issued into the two stages the
// previous pair used, then pair p is computed, so loads run two tiles ahead
// and the waves sharing a SIMD may drift apart by up to a tile between
// barriers.
template <int D>
__global__ void __launch_bounds__(DmaCfg<D>::THREADS, 2)
attn_wide_dma(AttnArgs a) {
  using C = DmaCfg<D>;
  // The ring: K stages 0..3, then V stages 0..3. Kept contiguous so that
  // every operand address is a lane base fixed for the launch plus an
  // immediate (the stage is known at compile time in the unrolled loop):
  // no per-tile address arithmetic.
  __shared__ __attribute__((aligned(1024))) char ring[8 * C::TB];
  char* const k0 = ring;
  char* const k1 = ring + C::TB;
  char* const k2 = ring + 2 * C::TB;
  char* const k3 = ring + 3 * C::TB;
  char* const v0 = ring + 4 * C::TB;
  char* const v1 = ring + 5 * C::TB;
  char* const v2 = ring + 6 * C::TB;
  char* const v3 = ring + 7 * C::TB;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, i = lane & 31, h = lane >> 5;
  const DmaLane<C> L = dma_lane<C>(wave, lane);
  RingLane<C> R;
#pragma unroll
  for (int q = 0; q < C::QF; ++q) {
    R.kaddr[q] = lds_u32(ring) + L.kaddr[q];
    asm volatile("" : "+v"(R.kaddr[q]));
  }
#pragma unroll
  for (int q = 0; q < C::OB; ++q) {
    R.vaddr[q] = lds_u32(ring) + 4 * C::TB + L.vaddr[q];
    asm volatile("" : "+v"(R.vaddr[q]));
  }
  const int bin_begin = a.bins[blockIdx.x], bin_end = a.bins[blockIdx.x + 1];
  State<C> s;   // carried from one item to the next along a chain
  for (int idx = bin_begin; idx < bin_end; ++idx) {
    // Every wave has finished reading the previous item's ring before its
    // stages are refilled.
    if (idx > bin_begin) lds_barrier();
    const WorkItem it = a.items[idx];
    const KvSrc<uint16_t> src = kv_src<uint16_t, D>(a, it, it.kv);
    const int kb0 = it.key_begin, ke = it.key_end;
    const int nt = (ke - kb0 + C::BN - 1) / C::BN;
    // The first pair's DMA goes out before the row bookkeeping and Q loads.
    dma_tile_any<C, D>(src, L, wave, kb0, ke, k0, v0);
    if (nt > 1) dma_tile_any<C, D>(src, L, wave, kb0 + C::BN, ke, k1, v1);
    const int rloc = wave * 32 + i;
    const Row w = row_at(a, it, rloc);
    // A chain's later shards continue from the state the previous item left
    // (ADR-0060, §4: the merge of two (m, l, O) states is the online
    // softmax's own update, done here in registers).
    if (!(it.chain & kChainContinues)) load_q<C, uint16_t, D>(a, w, it.kv, h, s);
    int pmin, pmax;
    wave_pos_range(w, &pmin, &pmax);
    const bool active = wave * 32 < it.n_rows;
    const float c = a.scale_log2;
#define GQA_RING_PAIR(SA, KN0, VN0, KN1, VN1)                                                               \
    {                                                                                                       \
      wait_dma<0>();                                                                                        \
      lds_barrier();                                                                                        \
      if (j + 2 < nt) dma_tile_any<C, D>(src, L, wave, kb0 + (j + 2) * C::BN, ke, KN0, VN0);                \
      if (j + 3 < nt) dma_tile_any<C, D>(src, L, wave, kb0 + (j + 3) * C::BN, ke, KN1, VN1);                \
      dma_step_ring<C, D, SA>(R, s, it.key_pos0, kb0 + j * C::BN, ke, a.causal, w.pos, pmin, pmax, active,  \
                              c, i, h);                                                                     \
      if (j + 1 < nt)                                                                                       \
        dma_step_ring<C, D, SA + 1>(R, s, it.key_pos0, kb0 + (j + 1) * C::BN, ke, a.causal, w.pos, pmin,    \
                                    pmax, active, c, i, h);                                                 \
    }
    for (int j0 = 0; j0 < nt; j0 += 4) {
      {
        const int j = j0;
        GQA_RING_PAIR(0, k2, v2, k3, v3)
      }
      if (j0 + 2 < nt) {
        const int j = j0 + 2;
        GQA_RING_PAIR(2, k0, v0, k1, v1)
      }
    }
#undef GQA_RING_PAIR
    if (!(it.chain & kChainContinued)) {
      s.l += __shfl_xor(s.l, 32);   // the two half-rows' sums, once per result
      write_row<C, uint16_t, D>(a, it, w, rloc, s.m, s.l, s.o, 0, C::OB, true, h);
    }
  }
}

// -------------------------------------------------------------- narrow ----
template <typename T, int D>
__global__ void __launch_bounds__(256, (Cfg<T, D, true>::WAVES_PER_SIMD))
attn_narrow(AttnArgs a) {
  using C = Cfg<T, D, true>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  __shared__ CombLds<C::BM> cl;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, i = lane & 31, h = lane >> 5;
  const int bin_begin = a.bins[blockIdx.x], bin_end = a.bins[blockIdx.x + 1];
  for (int idx = bin_begin; idx < bin_end; ++idx) {
    // Every wave has read the previous item's merge exchange before the
    // stages are refilled.
    if (idx > bin_begin) __syncthreads();
    const WorkItem it = a.items[idx];
    const Row w = row_at(a, it, i);
    State<C> s;
    load_q<C, T, D>(a, w, it.kv, h, s);
    combine_prepare(a, it, wave, lane, &cl);
    int pmin, pmax;
    wave_pos_range(w, &pmin, &pmax);
    const KvSrc<T> src = kv_src<T, D>(a, it, it.kv);

    const int nt = (it.key_end - it.key_begin + C::BN - 1) / C::BN;   // wave tiles: wave w takes w, w+4, ...
    const int rounds = (nt + 3) / 4;
    char* stg = smem + wave * C::STAGE;
    T* Ks = (T*)stg;
    T* Vs = (T*)(stg + C::K_ELEMS * sizeof(T));
    Stage<C> st;
    if (wave < nt) load_tile<C, T, D>(src, it.key_begin + wave * C::BN, it.key_end, lane, st);
    for (int rd = 0; rd < rounds; ++rd) {
      const int j = wave + 4 * rd;
      const bool have = j < nt;
      if (have) store_tile<C, T, D>(Ks, Vs, lane, st);
      __syncthreads();
      if (j + 4 < nt) load_tile<C, T, D>(src, it.key_begin + (j + 4) * C::BN, it.key_end, lane, st);
      if (have) {
        const int tk0 = it.key_begin + j * C::BN;
        const bool future = a.causal && (it.key_pos0 + tk0 > pmax);
        if (!future)
          run_tile<C, T, D>(Ks, Vs, s, it.key_pos0, tk0, it.key_end, a.causal, w.pos, pmin, a.scale_log2, i, h);
      }
      __syncthreads();
    }
    // Merge the four waves' states (same rows, disjoint keys) through LDS.
    float* mo = (float*)smem;                       // [wave][db][r][lane]
    float2* mml = (float2*)(smem + 4 * C::OB * 16 * 64 * 4);
#pragma unroll
    for (int db = 0; db < C::OB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) mo[((wave * C::OB + db) * 16 + r) * 64 + lane] = s.o[db][r];
    mml[wave * 64 + lane] = make_float2(s.m, s.l);
    __syncthreads();
    float mk[4], lk[4];
    float M = kNegInf;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float2 x = mml[k * 64 + lane];
      mk[k] = x.x;
      lk[k] = x.y;
      M = fmaxf(M, x.x);
    }
    const float M_use = (M == kNegInf) ? 0.f : M;
    float L = 0.f, wk[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      wk[k] = exp2_fast(mk[k] - M_use);
      L += lk[k] * wk[k];
    }
    for (int db = wave; db < C::OB; db += 4) {
      f32x16_t acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) x += wk[k] * mo[((k * C::OB + db) * 16 + r) * 64 + lane];
        acc[r] = x;
      }
      write_row<C, T, D>(a, it, w, i, M, L, &acc, db, db + 1, wave == 0, h);
    }
    combine_if_last<T, D, 256>(a, tid, &cl);
  }
}

// ---------------------------------------------------- narrow, bf16, DMA ----
// KV-bandwidth-bound items (<= 32 rows, decode): each of the 8 waves streams
// its own 32-key tiles (wave w takes tiles w, w+8, ...) through a private
// LDS stage filled by global->LDS DMA, with no barrier inside the loop. An
// item of up to 8 tiles (a 256-key shard) is requested in full at its start
// and each wave then computes a single tile, so little compute is left once
// the last bytes arrive. The eight per-wave (m, l, O) states are merged
// through LDS at the end. Same LDS swizzles, operand reads and softmax as
// the wide kernel.
template <int D>
struct NarrowDmaCfg {
  static constexpr bool BF16 = true;
  static constexpr int WAVES = 8;
  static constexpr int THREADS = 64 * WAVES;        // launch size (every launch and occupancy query uses it)
  static constexpr int BM = kNarrowRows;
  static constexpr int BN = 32;                     // keys per wave tile
  static constexpr int ROW = D * 2;
  static constexpr int TB = BN * ROW;               // bytes per tensor per tile
  static constexpr int NINST = TB / 1024;           // 1 KB DMA instructions per tensor per tile
  static constexpr int PER_WAVE = NINST;            // each wave issues its whole tile
  static constexpr int OB = D / 32, QF = D / 16, SB = BN / 32;
  static constexpr int MERGE_O = WAVES * OB * 16 * 64 * 4;   // bytes of the per-wave O^T exchange
  static_assert(WAVES * 2 * TB >= MERGE_O, "the stages must hold the merge exchange");
  static_assert(WAVES % OB == 0 && 4 % (WAVES / OB) == 0,
                "the waves split the O^T blocks' entry groups evenly in the final combination");
};

template <int D>
__global__ void __launch_bounds__(NarrowDmaCfg<D>::THREADS, 2)
attn_narrow_dma(AttnArgs a) {
  using C = NarrowDmaCfg<D>;
  __shared__ __attribute__((aligned(1024))) char st[C::WAVES * 2 * C::TB];   // per wave: K tile then V tile
  __shared__ float2 mml[C::WAVES * 64];
  __shared__ CombLds<C::BM> cl;
  __shared__ int pids[C::WAVES * 8];   // per wave: the page ids read ahead, parked during the tile's compute
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, i = lane & 31, h = lane >> 5;
  const DmaLane<C> L = dma_lane<C>(0, lane);
  const int bin_begin = a.bins[blockIdx.x], bin_end = a.bins[blockIdx.x + 1];
  for (int idx = bin_begin; idx < bin_end; ++idx) {
    // Every wave has read the previous item's merge exchange before the
    // stages are refilled.
    if (idx > bin_begin) __syncthreads();
    const WorkItem it = a.items[idx];
    const KvSrc<uint16_t> src = kv_src<uint16_t, D>(a, it, it.kv);
    const int kb0 = it.key_begin, ke = it.key_end, causal = a.causal;
    const int nt = (ke - kb0 + C::BN - 1) / C::BN;
    char* K0 = st + wave * 2 * C::TB;
    char* V0 = K0 + C::TB;
    // The row's token record and Q first, then the K/V stream: they need
    // only the work item, and loads issued behind a whole shard of K/V would
    // arrive last. The combination records are copied under the stream.
    const Row w = row_at(a, it, i);
    State<C> s;
    load_q<C, uint16_t, D>(a, w, it.kv, h, s);
    if (wave < nt) dma_tile_any<C, D>(src, L, 0, kb0 + wave * C::BN, ke, K0, V0);
    // Paged K/V: the page ids of the wave's next tile are read one step
    // ahead (page_ids_ahead), so its DMA can go out as soon as this tile's
    // stage is consumed.
    const bool ahead = src.paged && src.shift >= 4;
    int ids = 0;
    if (ahead && wave + C::WAVES < nt) ids = page_ids_ahead(src, kb0 + (wave + C::WAVES) * C::BN, ke, lane);
    combine_prepare(a, it, wave, lane, &cl);
    int pmin, pmax;
    wave_pos_range(w, &pmin, &pmax);
    const bool active = it.n_rows > 0;
    const float c = a.scale_log2;
    for (int j = wave; j < nt; j += C::WAVES) {
      wait_dma<0>();   // this tile, and the page ids of the next one
      if (ahead && lane < 8) pids[wave * 8 + lane] = ids;
      dma_step<C, D>(lds_u32(K0), lds_u32(V0), L, s, it.key_pos0, kb0 + j * C::BN, ke, causal, w.pos, pmin, pmax,
                     active, c, i, h);
      if (j + C::WAVES < nt) {
        wait_dma<63>();   // own LDS reads of the stage done
        const int key0n = kb0 + (j + C::WAVES) * C::BN;
        if (ahead) {
          const int parked = pids[wave * 8 + min(lane, 4)];
          int pg[5];
#pragma unroll
          for (int e = 0; e < 5; ++e) pg[e] = __builtin_amdgcn_readlane(parked, e);
          dma_tile<C, D, true, true, 3, true>(src, L, 0, key0n, ke, lds_u32(K0), lds_u32(V0), pg);
          if (j + 2 * C::WAVES < nt) ids = page_ids_ahead(src, key0n + C::WAVES * C::BN, ke, lane);
        } else {
          dma_tile_any<C, D>(src, L, 0, key0n, ke, K0, V0);
        }
      }
    }
    // Merge the eight waves' states (same rows, disjoint keys) through LDS:
    // only the lanes of the item's rows take part (a decode fills 8 of the
    // tile's 32), four accumulator entries per LDS access, and every wave
    // combines a quarter or half of one O^T block.
    s.l += __shfl_xor(s.l, 32);
    const RowDest dst = row_dest(a, it, w, i);
    // Addresses of this phase come from an opaque copy of the lane index, so
    // the compiler forms them here instead of hoisting them out of the item
    // loop, where they would hold registers through the K/V stream.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    wait_dma<0>();
    __syncthreads();
    float4* mo = (float4*)st;                     // [wave][db][group of 4 entries][lane]
    if (w.ok) {
#pragma unroll
      for (int db = 0; db < C::OB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          mo[((wave * C::OB + db) * 4 + r4) * 64 + ln] =
              make_float4(s.o[db][4 * r4], s.o[db][4 * r4 + 1], s.o[db][4 * r4 + 2], s.o[db][4 * r4 + 3]);
    }
    mml[wave * 64 + ln] = make_float2(s.m, s.l);
    __syncthreads();
    {
      constexpr int WPB = C::WAVES / C::OB, NQ = 4 / WPB;   // waves per O^T block, entry groups per wave
      const int db = wave / WPB, q0 = (wave % WPB) * NQ;
      float mk[C::WAVES], lk[C::WAVES];
      float M = kNegInf;
#pragma unroll
      for (int k = 0; k < C::WAVES; ++k) {
        const float2 x = mml[k * 64 + ln];
        mk[k] = x.x;
        lk[k] = x.y;
        M = fmaxf(M, x.x);
      }
      const float M_use = (M == kNegInf) ? 0.f : M;
      float Lsum = 0.f, wk[C::WAVES];
#pragma unroll
      for (int k = 0; k < C::WAVES; ++k) {
        wk[k] = exp2_fast(mk[k] - M_use);
        Lsum += lk[k] * wk[k];
      }
      float4 acc[NQ];
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (!w.ok) continue;
#pragma unroll
        for (int k = 0; k < C::WAVES; ++k) {
          const float4 v = mo[((k * C::OB + db) * 4 + q0 + j) * 64 + ln];
          acc[j].x += wk[k] * v.x;
          acc[j].y += wk[k] * v.y;
          acc[j].z += wk[k] * v.z;
          acc[j].w += wk[k] * v.w;
        }
      }
      if (a.coherent_parts)
        write_row_groups<uint16_t, D, true>(a, dst, w.ok, M, Lsum, acc, db, q0, wave == 0, h);
      else
        write_row_groups<uint16_t, D, false>(a, dst, w.ok, M, Lsum, acc, db, q0, wave == 0, h);
    }
    combine_if_last<uint16_t, D, C::THREADS>(a, tid, &cl);
  }
}

// --------------------------------------------------------------- merge ----
// One workgroup per (query token, KV head); each thread owns 4 consecutive
// d values of one of the G rows. Tokens whose partials all come from the
// narrow kernel were combined there (combine_if_last) and are skipped.
// Partials are folded in a fixed order (prefix shards, then suffix shards)
// with the same online rule as the tile loop, so the result is bitwise
// repeatable (ADR-0060 GQA fused attention, §4: m = max m_i, weights
// exp(m_i - m), normalise once at the end). Loads of several partials are
// issued before they are consumed.
template <typename T, int D, int U>
__global__ void __launch_bounds__(256)
lse_merge(AttnArgs a) {
  const int tok = blockIdx.x / a.H_kv, kv = blockIdx.x - tok * a.H_kv;
  const int ci = a.tok_rec[tok].comb;
  if (ci < 0) return;                    // single partial: written by the attention kernel
  const CombTok c = a.combs[ci];
  if (c.need > 0) return;                // combined inside the narrow launch
  constexpr int TPR = D / 4;   // threads per row
  const int n = c.live[0] + c.live[1];
  for (int g = threadIdx.x / TPR; g < a.G; g += 256 / TPR) {
    const int d0 = (threadIdx.x % TPR) * 4;
    float M = kNegInf, L = 0.f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
    fold_parts<D, U>(a, c, kv, g, 0, n, d0, M, L, O);
    write_combined<T, D>(a, tok, kv, g, d0, M, L, O);
  }
}

#define GQA_LAUNCH(KERNEL, GRID, BLOCK) \
  hipExtLaunchKernelGGL(KERNEL, dim3(GRID), dim3(BLOCK), 0, st, e0, e1, 0, a)

template <typename T, int D>
hipError_t launch_attn_t(const AttnArgs& a, int32_t n_bins, bool narrow, hipStream_t st, hipEvent_t e0,
                         hipEvent_t e1) {
  if (n_bins <= 0) return hipSuccess;
  if (narrow) {
    if constexpr (std::is_same<T, uint16_t>::value) GQA_LAUNCH((attn_narrow_dma<D>), n_bins, NarrowDmaCfg<D>::THREADS);
    else GQA_LAUNCH((attn_narrow<T, D>), n_bins, 256);
  } else if constexpr (std::is_same<T, uint16_t>::value) {
    GQA_LAUNCH((attn_wide_dma<D>), n_bins, DmaCfg<D>::THREADS);
  } else {
    GQA_LAUNCH((attn_wide<T, D>), n_bins, 256);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t occupancy_t(bool narrow, int* per_cu) {
  int n = 0;
  hipError_t e;
  if (narrow) {
    if constexpr (std::is_same<T, uint16_t>::value)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_narrow_dma<D>, NarrowDmaCfg<D>::THREADS, 0);
    else
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_narrow<T, D>, 256, 0);
  } else if constexpr (std::is_same<T, uint16_t>::value) {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_wide_dma<D>, DmaCfg<D>::THREADS, 0);
  } else {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_wide<T, D>, 256, 0);
  }
  *per_cu = n > 0 ? n : 1;
  return e;
}

// U = partials whose loads a thread issues before folding them: as many as
// the largest row needs (up to 16), fewer when rows have few partials so the
// kernel keeps its occupancy.
template <typename T, int D>
hipError_t launch_merge_t(const AttnArgs& a, int max_parts, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const int64_t blocks = (int64_t)a.n_q_tokens * a.H_kv;
  if (blocks <= 0) return hipSuccess;
  if (max_parts <= 4) GQA_LAUNCH((lse_merge<T, D, 4>), (unsigned)blocks, 256);
  else if (max_parts <= 8) GQA_LAUNCH((lse_merge<T, D, 8>), (unsigned)blocks, 256);
  else GQA_LAUNCH((lse_merge<T, D, 16>), (unsigned)blocks, 256);
  return hipGetLastError();
}
#undef GQA_LAUNCH

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int32_t n_bins, bool narrow, int dtype, int head_dim,
                            hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (dtype == 0) {
    if (head_dim == 128) return launch_attn_t<uint16_t, 128>(a, n_bins, narrow, stream, ev_start, ev_stop);
    return launch_attn_t<uint16_t, 64>(a, n_bins, narrow, stream, ev_start, ev_stop);
  }
  if (head_dim == 128) return launch_attn_t<float, 128>(a, n_bins, narrow, stream, ev_start, ev_stop);
  return launch_attn_t<float, 64>(a, n_bins, narrow, stream, ev_start, ev_stop);
}

hipError_t attention_occupancy(int dtype, int head_dim, bool narrow, int* per_cu) {
  if (dtype == 0) return head_dim == 128 ? occupancy_t<uint16_t, 128>(narrow, per_cu)
                                         : occupancy_t<uint16_t, 64>(narrow, per_cu);
  return head_dim == 128 ? occupancy_t<float, 128>(narrow, per_cu) : occupancy_t<float, 64>(narrow, per_cu);
}


hipError_t launch_merge(const AttnArgs& a, int dtype, int head_dim, int max_parts, hipStream_t stream,
                        hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (dtype == 0) {
    if (head_dim == 128) return launch_merge_t<uint16_t, 128>(a, max_parts, stream, ev_start, ev_stop);
    return launch_merge_t<uint16_t, 64>(a, max_parts, stream, ev_start, ev_stop);
  }
  if (head_dim == 128) return launch_merge_t<float, 128>(a, max_parts, stream, ev_start, ev_stop);
  return launch_merge_t<float, 64>(a, max_parts, stream, ev_start, ev_stop);
}

}  // namespace gqa
