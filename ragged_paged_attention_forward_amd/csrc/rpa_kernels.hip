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
//    are merged by log-sum-exp (by the last split to finish, or by
//    rpa_merge_kernel).
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
  int32_t* counters;     // one per split group, zero between calls
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;         // G = Hq / Hkv
  int32_t page_size;
  int32_t max_pages;
  int32_t window;
  float scale_log2;      // scale * log2(e)
  int32_t fused_merge;
};

// Element offset of key `t` of sequence row `pt_row` for KV head g.
RPA_DEV int64_t kv_offset(const int32_t* pt_row, int t, int page_size, int hkv, int g, int D) {
  const int page = pt_row[t / page_size];
  const int slot = t - (t / page_size) * page_size;
  return ((static_cast<int64_t>(page) * page_size + slot) * hkv + g) * D;
}

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

template <int D, int NB, int NW, int BN>
__global__ void __launch_bounds__(NW * 64)
rpa_prefill_kernel(KernelArgs args) {
  using C = PrefillCfg<D, NB, NW, BN>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* ks = smem;                  // [BN][KSTRIDE]
  uint16_t* vt = smem + C::LDS_K;       // [D][BN], swizzled 16-byte chunks

  const rpa_work_item it = args.items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 15;   // MFMA column: query row within a block; or key/d row
  const int lq = lane >> 4;   // lane quad 0..3

  const int hq = args.num_q_heads;
  const int hkv = args.num_kv_heads;
  const int G = args.group;
  const int g = it.kv_head;
  const int32_t* pt_row = args.page_table + static_cast<int64_t>(it.seq) * args.max_pages;

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
  const int n_tiles = (kv_end - kv_begin + BN - 1) / BN;
  const int pos_min = it.q_pos0;
  const int pos_max = it.q_pos0 + it.q_count - 1;
  const int window = args.window;
  const float sl2 = args.scale_log2;

  // ---- register staging of one K/V tile ----
  u32x4 kreg[C::K_PER_T];
  u32x4 vreg[C::V_PER_T][8];

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int u = i * C::NT + tid;
      kreg[i] = u32x4{0, 0, 0, 0};
      if (u < C::K_UNITS) {
        const int key = k0 + u / (D / 8);
        const int c = u % (D / 8);
        if (key < kv_end) kreg[i] = load16(args.k + kv_offset(pt_row, key, args.page_size, hkv, g, D) + c * 8);
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
        if (u < C::V_UNITS && key < kv_end)
          vreg[i][j] = load16(args.v + kv_offset(pt_row, key, args.page_size, hkv, g, D) + c * 8);
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

  if (n_tiles > 0) load_tile(kv_begin);

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int k0 = kv_begin + tile * BN;
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
    const bool full = (k0 + BN <= kv_end) && (k0 + BN - 1 <= pos_min) &&
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
// Split merge: out = sum_i 2^(lse_i - M) O_i / sum_i 2^(lse_i - M).
// One call merges one group; `tid`/`nthreads` stride over rows x D.
// ---------------------------------------------------------------------------
template <int D>
RPA_DEV void merge_group(const KernelArgs& args, const rpa_work_item& grp, int tid, int nthreads) {
  const int rows = grp.q_count * args.group;
  const int n = grp.num_splits;
  const float* lse = args.partial_lse + static_cast<int64_t>(grp.partial_base) * 16;
  const float* po = args.partial_o + static_cast<int64_t>(grp.partial_base) * 16 * D;
  constexpr int C4 = D / 4;
  for (int idx = tid; idx < rows * C4; idx += nthreads) {
    const int r = idx / C4;
    const int c = idx - r * C4;
    float mx = kNegInf;
    for (int i = 0; i < n; ++i) mx = fmaxf(mx, lse[i * 16 + r]);
    const float base = (mx == kNegInf) ? 0.f : mx;
    float wsum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < n; ++i) {
      const float w = fast_exp2(lse[i * 16 + r] - base);
      wsum += w;
      const f32x4 v = *reinterpret_cast<const f32x4*>(po + (static_cast<int64_t>(i) * 16 + r) * D + c * 4);
      acc += w * v;
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    acc *= inv;
    const int tk = r / args.group;
    const int hh = r - tk * args.group;
    uint16_t* dst = args.out + (static_cast<int64_t>(grp.q_start + tk) * args.num_q_heads +
                                grp.kv_head * args.group + hh) * D + c * 4;
    *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  }
}

template <int D>
__global__ void __launch_bounds__(256) rpa_merge_kernel(KernelArgs args) {
  const rpa_work_item grp = args.groups[blockIdx.x];
  merge_group<D>(args, grp, threadIdx.x, blockDim.x);
}

// ---------------------------------------------------------------------------
// Decode: rows = q_count * G <= 16; NW waves take 32-key chunks round robin.
// ---------------------------------------------------------------------------
template <int D>
struct DecodeCfg {
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int NCH = D / 8;                   // 16-byte chunks per key row
  static constexpr int NU = (NCH + 15) / 16;          // V chunk rounds per lane
  static constexpr int LDS_O = NW * 16 * D;           // floats
  static constexpr int LDS_BYTES = LDS_O * 4 + NW * 16 * 2 * 4;
};

template <int D>
__global__ void __launch_bounds__(256)
rpa_decode_kernel(KernelArgs args) {
  using C = DecodeCfg<D>;
  extern __shared__ __attribute__((aligned(16))) float dsm[];
  float* lds_o = dsm;                     // [NW][16][D]
  float* lds_m = dsm + C::LDS_O;          // [NW][16]
  float* lds_l = lds_m + C::NW * 16;      // [NW][16]
  __shared__ int s_last;

  const rpa_work_item it = args.items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 15;
  const int lq = lane >> 4;
  const int hq = args.num_q_heads;
  const int hkv = args.num_kv_heads;
  const int G = args.group;
  const int g = it.kv_head;
  const int rows = it.q_count * G;
  const int32_t* pt_row = args.page_table + static_cast<int64_t>(it.seq) * args.max_pages;
  const int kv_begin = it.kv_begin;
  const int kv_end = it.kv_end;
  const int window = args.window;
  const float sl2 = args.scale_log2;

  // row n = ln: token ln / G, head ln % G
  const int tk = ln / G;
  const int hh = ln - tk * G;
  const bool row_ok = ln < rows;
  const int pos = it.q_pos0 + tk;
  const int64_t row_off = (static_cast<int64_t>(it.q_start + tk) * hq + g * G + hh) * D;

  u32x4 qf[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    qf[kk] = row_ok ? load16(args.q + row_off + kk * 32 + lq * 8) : u32x4{0, 0, 0, 0};

  f32x4 o[C::NU][8];
#pragma unroll
  for (int u = 0; u < C::NU; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[u][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  const int n_chunks = (kv_end - kv_begin + 31) / 32;
  for (int ch = wave; ch < n_chunks; ch += C::NW) {
    const int k0 = kv_begin + ch * 32;
    // K rows k0 + 16*kb + ln, d = 32*kk + 8*lq (A operand of S^T = K Q^T)
    u32x4 kf[2][D / 32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = k0 + kb * 16 + ln;
      const bool ok = key < kv_end;
      const int64_t off = ok ? kv_offset(pt_row, key, args.page_size, hkv, g, D) : 0;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        kf[kb][kk] = ok ? load16(args.k + off + kk * 32 + lq * 8) : u32x4{0, 0, 0, 0};
    }
    // V rows: keys k0 + 4*lq + j and k0 + 16 + 4*lq + j at chunk 16*u + ln
    u32x4 vf[C::NU][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = k0 + ((j < 4) ? (lq * 4 + j) : (16 + lq * 4 + j - 4));
      const bool ok = key < kv_end;
      const int64_t off = ok ? kv_offset(pt_row, key, args.page_size, hkv, g, D) : 0;
#pragma unroll
      for (int u = 0; u < C::NU; ++u) {
        const int c = u * 16 + ln;
        vf[u][j] = (ok && c < C::NCH) ? load16(args.v + off + c * 8) : u32x4{0, 0, 0, 0};
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

  // ---- combine the waves through LDS ----
  const float l_wave = xor_sum(l_run);
  if (lq == 0) {
    lds_m[wave * 16 + ln] = m_run;
    lds_l[wave * 16 + ln] = l_wave;
  }
  // lane (lq, ln) holds O[row ln][d = 8*(16u + 4lq + j) + e]
#pragma unroll
  for (int u = 0; u < C::NU; ++u) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = u * 16 + lq * 4 + j;
      if (c < C::NCH) {
        float* dst = lds_o + (wave * 16 + ln) * D + c * 8;
        *reinterpret_cast<f32x4*>(dst) = f32x4{o[u][0][j], o[u][1][j], o[u][2][j], o[u][3][j]};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[u][4][j], o[u][5][j], o[u][6][j], o[u][7][j]};
      }
    }
  }
  __syncthreads();

  const bool split = it.split_group >= 0;
  const int64_t slot = static_cast<int64_t>(it.partial_base) + it.split_index;
  constexpr int C4 = D / 4;
  for (int idx = tid; idx < rows * C4; idx += C::NT) {
    const int r = idx / C4;
    const int c = idx - r * C4;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < C::NW; ++w) mx = fmaxf(mx, lds_m[w * 16 + r]);
    const float base = (mx == kNegInf) ? 0.f : mx;
    float lsum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < C::NW; ++w) {
      const float wt = fast_exp2(lds_m[w * 16 + r] - base);
      lsum += wt * lds_l[w * 16 + r];
      acc += wt * *reinterpret_cast<const f32x4*>(lds_o + (w * 16 + r) * D + c * 4);
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    acc *= inv;
    if (!split) {
      const int rtk = r / G;
      const int rhh = r - rtk * G;
      uint16_t* dst = args.out + (static_cast<int64_t>(it.q_start + rtk) * hq + g * G + rhh) * D + c * 4;
      *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    } else {
      *reinterpret_cast<f32x4*>(args.partial_o + (slot * 16 + r) * D + c * 4) = acc;
      if (c == 0) args.partial_lse[slot * 16 + r] = (lsum > 0.f) ? base + __builtin_log2f(lsum) : kNegInf;
    }
  }

  if (!split || !args.fused_merge) return;
  // Last split of the group to finish merges all of them.
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int prev = atomicAdd(args.counters + it.split_group, 1);
    s_last = (prev == it.num_splits - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  merge_group<D>(args, args.groups[it.split_group], tid, C::NT);
  if (tid == 0) atomicExch(args.counters + it.split_group, 0);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int D, int NB, int NW, int BN>
static hipError_t launch_prefill_t(const KernelArgs& a, int n_items, hipStream_t stream) {
  using C = PrefillCfg<D, NB, NW, BN>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&rpa_prefill_kernel<D, NB, NW, BN>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((rpa_prefill_kernel<D, NB, NW, BN>), dim3(n_items), dim3(C::NT), C::LDS_BYTES,
                     stream, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_t(const KernelArgs& a, int n_items, hipStream_t stream) {
  using C = DecodeCfg<D>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&rpa_decode_kernel<D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((rpa_decode_kernel<D>), dim3(n_items), dim3(C::NT), C::LDS_BYTES, stream, a);
  return hipGetLastError();
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
  a.counters = l.counters;
  a.num_q_heads = l.num_q_heads;
  a.num_kv_heads = l.num_kv_heads;
  a.group = l.num_q_heads / l.num_kv_heads;
  a.page_size = l.page_size;
  a.max_pages = l.max_pages;
  a.window = l.window;
  a.scale_log2 = l.scale_log2;
  a.fused_merge = l.fused_merge;
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
  switch (l.head_dim) {
    case 64: return launch_decode_t<64>(a, n_items, s);
    case 128: return launch_decode_t<128>(a, n_items, s);
    case 256: return launch_decode_t<256>(a, n_items, s);
    case 512: return launch_decode_t<512>(a, n_items, s);
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
