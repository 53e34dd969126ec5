// Ragged paged attention kernels for CDNA4 (gfx950).
//
// Two kernels consume the host-built work list:
//
//  * rpa_prefill_kernel -- one workgroup per (sequence, KV head, query tile)
//    item.  The tile packs NW*NB*16 rows of (token, query head of the KV
//    group) so every streamed key serves all grouped heads (the pages' kernel
//    scales its query block with the head ratio: "Chasing speed of light on
//    TPU v6e", footnote 6 of section Attention).  K/V pages are gathered by
//    coalesced 16-byte loads into LDS (V transposed on the way), the next tile
//    is fetched into registers while the current one is multiplied, and the
//    scores never leave the chip (footnote 5 of the same section).
//
//  * rpa_decode_kernel -- one workgroup per (sequence, KV head, key split) of
//    a sequence with few query rows (decode).  Decode is memory-bound at every
//    batch size ("TPU Deep Dive", chapter 4 and 7), so the waves of a
//    workgroup each stream a different 32-key chunk straight from HBM into
//    MFMA operand registers, and splits of long sequences run in parallel and
//    are merged by log-sum-exp in rpa_merge_kernel.
//
// Both compute S^T = K * Q^T and O^T = V^T * P^T with the bf16 MFMA
// v_mfma_f32_16x16x32_bf16, so that a query row is always the MFMA column
// index (lane % 16): row maxima, row sums and the O rescale stay within the
// four lanes {n, n+16, n+32, n+48} of row n.  Softmax runs in fp32 in base 2
// with log2(e) folded into the scale; the output is rounded to bf16 (RNE).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rpa.h"
#include "rpa_launch.h"

namespace rpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define RPA_DEV __device__ __forceinline__

constexpr float kNegInf = -__builtin_inff();

RPA_DEV f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

RPA_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

RPA_DEV float xor_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
RPA_DEV float xor_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// float -> bf16 bits, round to nearest even (NaN stays NaN).
RPA_DEV uint32_t bf16_bits(float f) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f)));
}
RPA_DEV uint32_t pack_bf16x2(float lo, float hi) { return bf16_bits(lo) | (bf16_bits(hi) << 16); }

// 8x8 transpose of 16-bit elements held as 8 rows of 16 bytes: out[e] holds
// element e of rows 0..7 (row j in half-word j).
RPA_DEV void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t a = in[2 * i][k];
      const uint32_t b = in[2 * i + 1][k];
      out[2 * k][i] = __builtin_amdgcn_perm(b, a, 0x05040100u);      // low halves
      out[2 * k + 1][i] = __builtin_amdgcn_perm(b, a, 0x07060302u);  // high halves
    }
  }
}

RPA_DEV u32x4 load16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// Wave-uniform load through the constant address space, so it becomes a
// scalar load that does not wait behind the vector loads in flight.
typedef const int32_t __attribute__((address_space(4)))* const_i32_ptr;
RPA_DEV int32_t uniform_load(const int32_t* p, int idx) {
  return ((const_i32_ptr)(p))[idx];
}

struct KernelArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* page_table;
  uint16_t* out;
  const rpa_work_item* items;
  const rpa_work_item* groups;
  float* partial_o;      // [slot][16 rows][D]
  float* partial_lse;    // [slot][16 rows], base-2 log-sum-exp
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;         // G = Hq / Hkv
  int32_t page_size;
  int32_t max_pages;
  int32_t window;
  float scale_log2;      // scale * log2(e)
};

RPA_DEV bool key_visible(int key, int pos, int kv_begin, int kv_end, int window) {
  return key >= kv_begin && key < kv_end && key <= pos && (window <= 0 || key > pos - window);
}

// ---------------------------------------------------------------------------
// Prefill: NW waves x NB row blocks of 16 rows; BN keys per LDS tile.
// ---------------------------------------------------------------------------
template <int D, int NB, int NW, int BN>
struct PrefillCfg {
  static constexpr int NT = NW * 64;
  static constexpr int KSTRIDE = D + 8;            // bf16 elements per K row in LDS (padded)
  static constexpr int NCHUNK = BN / 8;            // 16-byte chunks per V^T row
  static constexpr int K_UNITS = BN * (D / 8);     // 16-byte K pieces per tile
  static constexpr int K_PER_T = (K_UNITS + NT - 1) / NT;
  static constexpr int V_UNITS = (BN / 32) * 4 * (D / 8);  // 8-key x 16-byte V pieces
  static constexpr int V_PER_T = (V_UNITS + NT - 1) / NT;
  static constexpr int LDS_K = BN * KSTRIDE;       // bf16 elements
  static constexpr int LDS_V = D * BN;
  static constexpr int LDS_BYTES = (LDS_K + LDS_V) * 2;
  static_assert(BN % 32 == 0, "BN must be a multiple of 32");
  static_assert(D % 32 == 0, "D must be a multiple of 32");
};

// Swizzled 16-byte chunk of V^T row r: spreads both the transposed writes
// (rows 8 apart) and the MFMA operand reads (consecutive rows) over the banks.
template <int BN>
RPA_DEV int vt_chunk(int r, int chunk) {
  constexpr int NC = BN / 8;
  const int sw = (NC >= 8) ? (r ^ (r >> 3)) : ((r >> 1) ^ (r >> 3));
  return chunk ^ (sw & (NC - 1));
}

template <int D, int NB, int NW, int BN, bool UNI>
__global__ void __launch_bounds__(NW * 64)
rpa_prefill_kernel(KernelArgs args) {
  using C = PrefillCfg<D, NB, NW, BN>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* ks = smem;                  // [BN][KSTRIDE]
  uint16_t* vt = smem + C::LDS_K;       // [D][BN], swizzled 16-byte chunks

  const rpa_work_item it = args.items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int ln = lane & 15;   // MFMA column: query row within a block; or key/d row
  const int lq = lane >> 4;   // lane quad 0..3

  const int hq = args.num_q_heads;
  const int hkv = args.num_kv_heads;
  const int G = args.group;
  const int g = it.kv_head;
  const int32_t* __restrict__ pt_row = args.page_table + static_cast<int64_t>(it.seq) * args.max_pages;
  const uint16_t* __restrict__ kbase = args.k;
  const uint16_t* __restrict__ vbase = args.v;
  const int page_size = args.page_size;
  const int64_t row_stride = static_cast<int64_t>(hkv) * D;  // elements between slots of a page

  // ---- per-lane rows, Q fragments (B operand of S^T = K Q^T) ----
  int row_pos[NB];
  bool row_ok[NB];
  int64_t row_off[NB];  // element offset of (token, head) row in q/out
  u32x4 qf[NB][D / 32];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r = (wave * NB + nb) * 16 + ln;
    const int tk = r / G;
    const int hh = r - tk * G;
    row_ok[nb] = tk < it.q_count;
    row_pos[nb] = it.q_pos0 + tk;
    row_off[nb] = (static_cast<int64_t>(it.q_start + tk) * hq + g * G + hh) * D;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      qf[nb][kk] = row_ok[nb] ? load16(args.q + row_off[nb] + kk * 32 + lq * 8) : u32x4{0, 0, 0, 0};
    }
  }

  f32x4 o[D / 16][NB];
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[db][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = kNegInf;
    l_run[nb] = 0.f;
  }

  const int kv_begin = it.kv_begin;
  const int kv_end = it.kv_end;
  const int tile0 = (kv_begin / BN) * BN;  // tiles are aligned to BN keys
  const int n_tiles = (kv_end - tile0 + BN - 1) / BN;
  const int pos_min = it.q_pos0;
  const int pos_max = it.q_pos0 + it.q_count - 1;
  const int window = args.window;
  const float sl2 = args.scale_log2;

  // ---- register staging of one K/V tile ----
  u32x4 kreg[C::K_PER_T];
  u32x4 vreg[C::V_PER_T][8];

  // Element offset of key `key` (KV head g).  With UNI every page holds a whole
  // number of tiles, so one wave-uniform page lookup serves the tile.
  auto load_tile = [&](int k0) {
    int64_t ubase = 0;
    if constexpr (UNI) {
      const int pidx = k0 / page_size;
      const int64_t page = uniform_load(pt_row, pidx);
      ubase = ((page * page_size + (k0 - pidx * page_size)) * hkv + g) * D;
    }
    auto kv_row = [&](int key, int pid) -> int64_t {
      if constexpr (UNI) {
        return ubase + static_cast<int64_t>(key - k0) * row_stride;
      } else {
        const int slot = key - (key / page_size) * page_size;
        return ((static_cast<int64_t>(pid) * page_size + slot) * hkv + g) * D;
      }
    };
    // page ids of every row this thread loads, fetched before any K/V load
    int kpid[C::K_PER_T];
    int vpid[C::V_PER_T][8];
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      kpid[i] = 0;
      if constexpr (!UNI) {
        const int u = i * C::NT + tid;
        const int key = k0 + u / (D / 8);
        if (u < C::K_UNITS && key >= kv_begin && key < kv_end) kpid[i] = pt_row[key / page_size];
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
      const int u = i * C::NT + tid;
      const int grp = u / (D / 8);
      const int t = grp >> 2;
      const int qd = grp & 3;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        vpid[i][j] = 0;
        if constexpr (!UNI) {
          const int key = k0 + t * 32 + ((j < 4) ? (qd * 4 + j) : (16 + qd * 4 + j - 4));
          if (u < C::V_UNITS && key >= kv_begin && key < kv_end) vpid[i][j] = pt_row[key / page_size];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int u = i * C::NT + tid;
      kreg[i] = u32x4{0, 0, 0, 0};
      if (u < C::K_UNITS) {
        const int key = k0 + u / (D / 8);
        const int c = u % (D / 8);
        if (key >= kv_begin && key < kv_end) kreg[i] = load16(kbase + kv_row(key, kpid[i]) + c * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
      const int u = i * C::NT + tid;
      const int c = u % (D / 8);
      const int grp = u / (D / 8);      // (t, quad) pair
      const int t = grp >> 2;
      const int qd = grp & 3;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        vreg[i][j] = u32x4{0, 0, 0, 0};
        const int key = k0 + t * 32 + ((j < 4) ? (qd * 4 + j) : (16 + qd * 4 + j - 4));
        if (u < C::V_UNITS && key >= kv_begin && key < kv_end)
          vreg[i][j] = load16(vbase + kv_row(key, vpid[i][j]) + c * 8);
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int u = i * C::NT + tid;
      if (u < C::K_UNITS) {
        const int key = u / (D / 8);
        const int c = u % (D / 8);
        *reinterpret_cast<u32x4*>(ks + key * C::KSTRIDE + c * 8) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_T; ++i) {
      const int u = i * C::NT + tid;
      if (u < C::V_UNITS) {
        const int c = u % (D / 8);
        const int grp = u / (D / 8);
        u32x4 tr[8];
        transpose8x8(vreg[i], tr);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = c * 8 + e;  // d index = V^T row
          *reinterpret_cast<u32x4*>(vt + r * BN + vt_chunk<BN>(r, grp) * 8) = tr[e];
        }
      }
    }
  };

  if (n_tiles > 0) load_tile(tile0);

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int k0 = tile0 + tile * BN;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (tile + 1 < n_tiles) load_tile(k0 + BN);

    // ---- S^T = K Q^T ----
    f32x4 s[BN / 16][NB];
#pragma unroll
    for (int kb = 0; kb < BN / 16; ++kb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[kb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(ks + (kb * 16 + ln) * C::KSTRIDE + kk * 32 + lq * 8);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s[kb][nb] = mfma16(a, qf[nb][kk], s[kb][nb]);
      }
    }

    // ---- mask + online softmax (fp32, base 2) ----
    const bool full = (k0 >= kv_begin) && (k0 + BN <= kv_end) && (k0 + BN - 1 <= pos_min) &&
                      (window <= 0 || k0 > pos_max - window);
    u32x4 pf[BN / 32][NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float x = s[kb][nb][j] * sl2;
          if (!full) {
            const int key = k0 + kb * 16 + lq * 4 + j;
            if (!key_visible(key, row_pos[nb], kv_begin, kv_end, window)) x = kNegInf;
          }
          s[kb][nb][j] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = xor_max(mx);
      const float m_new = fmaxf(m_run[nb], mx);
      const float base = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[nb] - base);
      m_run[nb] = m_new;
      float lsum = 0.f;
#pragma unroll
      for (int t = 0; t < BN / 32; ++t) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[j] = fast_exp2(s[2 * t][nb][j] - base);
          p[4 + j] = fast_exp2(s[2 * t + 1][nb][j] - base);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) lsum += p[j];
        pf[t][nb] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                          pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
      }
      l_run[nb] = l_run[nb] * alpha + lsum;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) o[db][nb] *= alpha;
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int t = 0; t < BN / 32; ++t) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const int r = db * 16 + ln;
        const u32x4 a = *reinterpret_cast<const u32x4*>(vt + r * BN + vt_chunk<BN>(r, t * 4 + lq) * 8);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) o[db][nb] = mfma16(a, pf[t][nb], o[db][nb]);
      }
    }
  }

  // ---- epilogue: O / l -> bf16 ----
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float l = xor_sum(l_run[nb]);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (row_ok[nb]) {
      uint16_t* dst = args.out + row_off[nb] + lq * 4;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const f32x4 v = o[db][nb] * inv;
        *reinterpret_cast<u32x2*>(dst + db * 16) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split merge: out = sum_i 2^(lse_i - M) O_i / sum_i 2^(lse_i - M), M = max_i lse_i.
// One workgroup per group; each thread owns one 4-float column of one row.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) rpa_merge_kernel(KernelArgs args) {
  const rpa_work_item grp = args.groups[blockIdx.x];
  constexpr int C4 = D / 4;
  const int rows = grp.q_count * args.group;
  const int n = grp.num_splits;
  const float* lse = args.partial_lse + static_cast<int64_t>(grp.partial_base) * 16;
  const float* po = args.partial_o + static_cast<int64_t>(grp.partial_base) * 16 * D;
  for (int idx = threadIdx.x; idx < rows * C4; idx += blockDim.x) {
    const int r = idx / C4;
    const int c = idx - r * C4;
    float mx = kNegInf;
    for (int i = 0; i < n; ++i) mx = fmaxf(mx, lse[i * 16 + r]);
    const float base = (mx == kNegInf) ? 0.f : mx;
    float wsum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int i = 0; i < n; ++i) {
      const float w = fast_exp2(lse[i * 16 + r] - base);
      const f32x4 v = *reinterpret_cast<const f32x4*>(po + (static_cast<int64_t>(i) * 16 + r) * D + c * 4);
      wsum += w;
      acc += w * v;
    }
    acc *= wsum > 0.f ? 1.f / wsum : 0.f;
    const int tk = r / args.group;
    const int hh = r - tk * args.group;
    uint16_t* dst = args.out + (static_cast<int64_t>(grp.q_start + tk) * args.num_q_heads +
                                grp.kv_head * args.group + hh) * D + c * 4;
    *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  }
}

// ---------------------------------------------------------------------------
// Decode: rows = q_count * G <= 16; NW waves take 32-key chunks round robin.
// Every wave issues all loads of a chunk before touching any of them; the
// waves are combined in a fixed order through LDS (bitwise reproducible).
// ---------------------------------------------------------------------------
template <int D, int NW>
struct DecodeCfg {
  static constexpr int NT = NW * 64;
  static constexpr int NCH = D / 8;                   // 16-byte chunks per key row
  static constexpr int NU = (NCH + 15) / 16;          // V chunk rounds per lane
  static constexpr int OSTRIDE = D + 4;               // floats per LDS row (padded)
  static constexpr int LDS_O = (NW / 2) * 16 * OSTRIDE; // tree-combine slots
  static constexpr int LDS_BYTES = LDS_O * 4 + NW * 16 * 2 * 4;
};

// Second launch bound: waves per SIMD to fit (two, so a compute unit holds two
// workgroups of 4 waves; one for D = 512 whose fragments need the full file).
template <int D, int NW, bool UNI>
__global__ void __launch_bounds__(NW * 64, D >= 512 ? 1 : 2)
rpa_decode_kernel(KernelArgs args) {
  using C = DecodeCfg<D, NW>;
  extern __shared__ __attribute__((aligned(16))) float dsm[];
  float* lds_o = dsm;                     // [NW/2][16][OSTRIDE]
  float* lds_m = dsm + C::LDS_O;          // [NW][16]
  float* lds_l = lds_m + NW * 16;         // [NW][16]

  const rpa_work_item it = args.items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int ln = lane & 15;
  const int lq = lane >> 4;
  const int hq = args.num_q_heads;
  const int hkv = args.num_kv_heads;
  const int G = args.group;
  const int g = it.kv_head;
  const int rows = it.q_count * G;
  const int32_t* __restrict__ pt_row = args.page_table + static_cast<int64_t>(it.seq) * args.max_pages;
  const uint16_t* __restrict__ kbase = args.k;
  const uint16_t* __restrict__ vbase = args.v;
  const int page_size = args.page_size;
  const int64_t row_stride = static_cast<int64_t>(hkv) * D;
  const int kv_begin = it.kv_begin;
  const int kv_end = it.kv_end;
  const int window = args.window;
  const float sl2 = args.scale_log2;

  // query row n = ln: token ln / G, head ln % G
  const int tk = ln / G;
  const int hh = ln - tk * G;
  const bool row_ok = ln < rows;
  const int pos = it.q_pos0 + tk;
  const int64_t q_off = (static_cast<int64_t>(it.q_start + tk) * hq + g * G + hh) * D;

  u32x4 qf[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    qf[kk] = row_ok ? load16(args.q + q_off + kk * 32 + lq * 8) : u32x4{0, 0, 0, 0};

  f32x4 o[C::NU][8];
#pragma unroll
  for (int u = 0; u < C::NU; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[u][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  // 32-key chunks aligned to 32 keys; with UNI a chunk never crosses a page.
  const int chunk0 = (kv_begin / 32) * 32;
  const int n_chunks = (kv_end - chunk0 + 31) / 32;
  for (int ch = wave; ch < n_chunks; ch += NW) {
    const int k0 = chunk0 + ch * 32;
    int64_t ubase = 0;
    if constexpr (UNI) {
      const int pidx = k0 / page_size;
      const int64_t page = uniform_load(pt_row, pidx);
      ubase = ((page * page_size + (k0 - pidx * page_size)) * hkv + g) * D;
    }
    // keys of this lane: K rows k0 + 16*kb + ln; V rows k0 + 4*lq + j and k0 + 16 + 4*lq + j
    int kkey[2], vkey[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) kkey[kb] = k0 + kb * 16 + ln;
#pragma unroll
    for (int j = 0; j < 8; ++j) vkey[j] = k0 + ((j < 4) ? (lq * 4 + j) : (16 + lq * 4 + j - 4));
    int kpid[2] = {0, 0}, vpid[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (!UNI) {   // every page id first, then the K/V loads
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kkey[kb] >= kv_begin && kkey[kb] < kv_end) kpid[kb] = pt_row[kkey[kb] / page_size];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (vkey[j] >= kv_begin && vkey[j] < kv_end) vpid[j] = pt_row[vkey[j] / page_size];
    }
    auto kv_row = [&](int key, int pid) -> int64_t {
      if constexpr (UNI) {
        return ubase + static_cast<int64_t>(key - k0) * row_stride;
      } else {
        const int slot = key - (key / page_size) * page_size;
        return ((static_cast<int64_t>(pid) * page_size + slot) * hkv + g) * D;
      }
    };
    // K rows (A operand of S^T = K Q^T): d = 32*kk + 8*lq
    u32x4 kf[2][D / 32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bool ok = kkey[kb] >= kv_begin && kkey[kb] < kv_end;
      const int64_t off = kv_row(kkey[kb], kpid[kb]);
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        kf[kb][kk] = ok ? load16(kbase + off + kk * 32 + lq * 8) : u32x4{0, 0, 0, 0};
    }
    // V rows at 16-byte chunk 16*u + ln
    u32x4 vf[C::NU][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool ok = vkey[j] >= kv_begin && vkey[j] < kv_end;
      const int64_t off = kv_row(vkey[j], vpid[j]);
#pragma unroll
      for (int u = 0; u < C::NU; ++u) {
        const int c = u * 16 + ln;
        vf[u][j] = (ok && c < C::NCH) ? load16(vbase + off + c * 8) : u32x4{0, 0, 0, 0};
      }
    }

    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) s[kb] = mfma16(kf[kb][kk], qf[kk], s[kb]);
    }

    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = k0 + kb * 16 + lq * 4 + j;
        float x = s[kb][j] * sl2;
        if (!key_visible(key, pos, kv_begin, kv_end, window)) x = kNegInf;
        s[kb][j] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = xor_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float base = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - base);
    m_run = m_new;
    float p[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] = fast_exp2(s[0][j] - base);
      p[4 + j] = fast_exp2(s[1][j] - base);
    }
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) lsum += p[j];
    l_run = l_run * alpha + lsum;
    const u32x4 pf = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                      pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
#pragma unroll
    for (int u = 0; u < C::NU; ++u) {
      u32x4 vt[8];
      transpose8x8(vf[u], vt);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[u][e] = mfma16(vt[e], pf, o[u][e] * alpha);
    }
  }

  // ---- combine the waves: common max, per-wave weight, fixed-order tree ----
  const float l_wave = xor_sum(l_run);
  if (lq == 0) {
    lds_m[wave * 16 + ln] = m_run;
    lds_l[wave * 16 + ln] = l_wave;
  }
  __syncthreads();
  float mx = kNegInf;
#pragma unroll
  for (int w = 0; w < NW; ++w) mx = fmaxf(mx, lds_m[w * 16 + ln]);
  const float base = (mx == kNegInf) ? 0.f : mx;
  float lsum = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) lsum += fast_exp2(lds_m[w * 16 + ln] - base) * lds_l[w * 16 + ln];
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const float wscale = fast_exp2(m_run - base) * inv;   // this wave's share, normalised
#pragma unroll
  for (int u = 0; u < C::NU; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[u][e] *= wscale;
  // lane (lq, ln) holds O[row ln][d = 8*(16u + 4lq + j) + e]; slot rows are padded by 4 floats
  auto slot_ptr = [&](int slot, int u, int j) {
    return reinterpret_cast<f32x4*>(lds_o + (slot * 16 + ln) * C::OSTRIDE + (u * 16 + lq * 4 + j) * 8);
  };
#pragma unroll
  for (int half = NW / 2; half >= 1; half /= 2) {
    if (wave >= half && wave < 2 * half && row_ok) {
#pragma unroll
      for (int u = 0; u < C::NU; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (u * 16 + lq * 4 + j < C::NCH) {
            f32x4* dst = slot_ptr(wave - half, u, j);
            dst[0] = f32x4{o[u][0][j], o[u][1][j], o[u][2][j], o[u][3][j]};
            dst[1] = f32x4{o[u][4][j], o[u][5][j], o[u][6][j], o[u][7][j]};
          }
    }
    __syncthreads();
    if (wave < half && row_ok) {
#pragma unroll
      for (int u = 0; u < C::NU; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (u * 16 + lq * 4 + j < C::NCH) {
            const f32x4* src = slot_ptr(wave, u, j);
            const f32x4 lo = src[0], hi = src[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              o[u][e][j] += lo[e];
              o[u][4 + e][j] += hi[e];
            }
          }
    }
    if (half > 1) __syncthreads();
  }
  if (wave != 0 || !row_ok) return;

  // ---- wave 0 writes the output row (or the split's partial) from registers ----
  const bool split = it.split_group >= 0;
  if (!split) {
    uint16_t* dst = args.out + q_off;
#pragma unroll
    for (int u = 0; u < C::NU; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = u * 16 + lq * 4 + j;
        if (c < C::NCH)
          *reinterpret_cast<u32x4*>(dst + c * 8) =
              u32x4{pack_bf16x2(o[u][0][j], o[u][1][j]), pack_bf16x2(o[u][2][j], o[u][3][j]),
                    pack_bf16x2(o[u][4][j], o[u][5][j]), pack_bf16x2(o[u][6][j], o[u][7][j])};
      }
  } else {
    const int64_t slot = static_cast<int64_t>(it.partial_base) + it.split_index;
    float* dst = args.partial_o + (slot * 16 + ln) * D;
#pragma unroll
    for (int u = 0; u < C::NU; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = u * 16 + lq * 4 + j;
        if (c < C::NCH) {
          *reinterpret_cast<f32x4*>(dst + c * 8) = f32x4{o[u][0][j], o[u][1][j], o[u][2][j], o[u][3][j]};
          *reinterpret_cast<f32x4*>(dst + c * 8 + 4) = f32x4{o[u][4][j], o[u][5][j], o[u][6][j], o[u][7][j]};
        }
      }
    if (lq == 0) args.partial_lse[slot * 16 + ln] = (lsum > 0.f) ? base + __builtin_log2f(lsum) : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int D, int NB, int NW, int BN, bool UNI>
static hipError_t launch_prefill_u(const KernelArgs& a, int n_items, hipStream_t stream) {
  using C = PrefillCfg<D, NB, NW, BN>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&rpa_prefill_kernel<D, NB, NW, BN, UNI>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((rpa_prefill_kernel<D, NB, NW, BN, UNI>), dim3(n_items), dim3(C::NT), C::LDS_BYTES,
                     stream, a);
  return hipGetLastError();
}

template <int D, int NB, int NW, int BN>
static hipError_t launch_prefill_t(const KernelArgs& a, int n_items, hipStream_t stream) {
  if (a.page_size % BN == 0) return launch_prefill_u<D, NB, NW, BN, true>(a, n_items, stream);
  return launch_prefill_u<D, NB, NW, BN, false>(a, n_items, stream);
}

template <int D, int NW, bool UNI>
static hipError_t launch_decode_u(const KernelArgs& a, int n_items, hipStream_t stream) {
  using C = DecodeCfg<D, NW>;
  hipLaunchKernelGGL((rpa_decode_kernel<D, NW, UNI>), dim3(n_items), dim3(C::NT), C::LDS_BYTES, stream, a);
  return hipGetLastError();
}

// Eight-wave workgroups are not used for D = 512: two waves per SIMD cannot
// hold its fragments.
template <int D>
static hipError_t launch_decode_t(const KernelArgs& a, int n_items, int waves, hipStream_t stream) {
  const bool uni = a.page_size % 32 == 0;
  if (waves == 8 && D < 512) return uni ? launch_decode_u<D, 8, true>(a, n_items, stream)
                             : launch_decode_u<D, 8, false>(a, n_items, stream);
  return uni ? launch_decode_u<D, 4, true>(a, n_items, stream) : launch_decode_u<D, 4, false>(a, n_items, stream);
}

template <int D>
static hipError_t launch_merge_t(const KernelArgs& a, int n_groups, hipStream_t stream) {
  hipLaunchKernelGGL((rpa_merge_kernel<D>), dim3(n_groups), dim3(256), 0, stream, a);
  return hipGetLastError();
}

int prefill_rows_for(int head_dim) {
  switch (head_dim) {
    case 64: return 4 * 2 * 16;
    case 128: return 4 * 2 * 16;
    case 256: return 4 * 2 * 16;
    case 512: return 4 * 1 * 16;
    default: return 0;
  }
}

bool head_dim_supported(int head_dim) { return prefill_rows_for(head_dim) > 0; }

static KernelArgs make_args(const LaunchArgs& l, const rpa_work_item* items) {
  KernelArgs a;
  a.q = static_cast<const uint16_t*>(l.q);
  a.k = static_cast<const uint16_t*>(l.k);
  a.v = static_cast<const uint16_t*>(l.v);
  a.page_table = l.page_table;
  a.out = static_cast<uint16_t*>(l.out);
  a.items = items;
  a.groups = l.groups;
  a.partial_o = l.partial_o;
  a.partial_lse = l.partial_lse;
  a.num_q_heads = l.num_q_heads;
  a.num_kv_heads = l.num_kv_heads;
  a.group = l.num_q_heads / l.num_kv_heads;
  a.page_size = l.page_size;
  a.max_pages = l.max_pages;
  a.window = l.window;
  a.scale_log2 = l.scale_log2;
  return a;
}

hipError_t launch_prefill(const LaunchArgs& l, const rpa_work_item* items, int n_items) {
  if (n_items <= 0) return hipSuccess;
  const KernelArgs a = make_args(l, items);
  hipStream_t s = static_cast<hipStream_t>(l.stream);
  switch (l.head_dim) {
    case 64: return launch_prefill_t<64, 2, 4, 64>(a, n_items, s);
    case 128: return launch_prefill_t<128, 2, 4, 64>(a, n_items, s);
    case 256: return launch_prefill_t<256, 2, 4, 64>(a, n_items, s);
    case 512: return launch_prefill_t<512, 1, 4, 32>(a, n_items, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const LaunchArgs& l, const rpa_work_item* items, int n_items) {
  if (n_items <= 0) return hipSuccess;
  const KernelArgs a = make_args(l, items);
  hipStream_t s = static_cast<hipStream_t>(l.stream);
  const int w = l.decode_waves;
  switch (l.head_dim) {
    case 64: return launch_decode_t<64>(a, n_items, w, s);
    case 128: return launch_decode_t<128>(a, n_items, w, s);
    case 256: return launch_decode_t<256>(a, n_items, w, s);
    case 512: return launch_decode_t<512>(a, n_items, w, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_merge(const LaunchArgs& l, int n_groups) {
  if (n_groups <= 0) return hipSuccess;
  const KernelArgs a = make_args(l, nullptr);
  hipStream_t s = static_cast<hipStream_t>(l.stream);
  switch (l.head_dim) {
    case 64: return launch_merge_t<64>(a, n_groups, s);
    case 128: return launch_merge_t<128>(a, n_groups, s);
    case 256: return launch_merge_t<256>(a, n_groups, s);
    case 512: return launch_merge_t<512>(a, n_groups, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rpa
