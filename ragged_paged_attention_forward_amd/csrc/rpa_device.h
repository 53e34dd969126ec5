// Device code of the ragged paged attention kernels (included by one
// translation unit per head size, see rpa_kernels_d*.hip).
#pragma once
// Ragged paged attention kernels for CDNA4 (gfx950).
//
// Two kernels consume the host-built work list:
//
//  * rpa_prefill_kernel -- one workgroup per (sequence, KV head, query tile)
//    item.  The tile packs (NW/DS)*NB*32 rows of (token, query head of the KV
//    group), so every streamed key serves all grouped heads (the pages'
//    kernel scales its query block with the head ratio: "Chasing speed of
//    light on TPU v6e", footnote 6 of section Attention).  K/V tiles of BN
//    keys go from HBM straight into NS LDS buffers (buffer loads with an LDS
//    destination, XOR-swizzled rows), in a rotated order that lets
//    neighbouring query tiles share them through the L2; S^T = K Q^T and
//    O^T += V^T P^T run on v_mfma_f32_32x32x16_bf16 with V^T read by
//    transposing LDS reads, and the scores never leave the chip (footnote 5
//    of the same section).
//
//  * rpa_decode_kernel -- one workgroup per (sequence, KV head, key split) of
//    a sequence with few query rows (decode).  Decode is memory-bound at every
//    batch size ("TPU Deep Dive", chapter 4 and 7), so the waves of a
//    workgroup each stream a different 32-key chunk straight from HBM into
//    v_mfma_f32_16x16x32_bf16 operand registers; the waves are combined
//    through LDS, and the splits of a long sequence are merged by log-sum-exp
//    by the split that finishes last (or by rpa_merge_kernel, which always
//    merges the splits of long prefill items).
//
// Both compute scores transposed (S^T = K Q^T), so a query row is an MFMA
// column and the probabilities feed the P V product from the same lanes.
// Softmax runs in fp32 in base 2 with log2(e) folded into the scale; the
// output is rounded to bf16 (round to nearest even).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rpa.h"
#include "rpa_launch.h"
#include "rpa_kargs.h"

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

// Two floats -> packed bf16 pair (lo in bits 0-15), round to nearest even,
// NaN stays NaN: one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
RPA_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
// The same rounding, one value at a time (the decode kernel's register
// allocation fares better with this form).
RPA_DEV uint32_t pack_bf16x2_split(float lo, float hi) {
  const uint32_t a = __builtin_bit_cast(uint16_t, static_cast<__bf16>(lo));
  const uint32_t b = __builtin_bit_cast(uint16_t, static_cast<__bf16>(hi));
  return a | (b << 16);
}

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

// Buffer resource over `bytes` bytes from `base` (gfx9 descriptor: 32-bit data
// format, raw addressing).  Loads at offsets at or past `bytes` -- including
// negative offsets, which wrap to huge unsigned values -- return zero.
RPA_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                          static_cast<int>(bytes), 0x00020000);
}
RPA_DEV u32x4 buffer_load16(__amdgpu_buffer_rsrc_t rs, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 0));
}

RPA_DEV u32x2 load8(const uint8_t* p) { return *reinterpret_cast<const u32x2*>(p); }
RPA_DEV u32x4 load16b(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }
RPA_DEV u32x2 buffer_load8(__amdgpu_buffer_rsrc_t rs, int byte_off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, byte_off, 0, 0));
}

// Eight OCP FP8 E4M3 bytes (two little-endian words) to the eight bf16 a
// 16-byte load of bf16 elements would give (element i in half-word i).
// Every E4M3 value is exact in bf16; v_cvt_scalef32_pk_bf16_fp8 with scale
// 1.0 converts the low or the high byte pair of a word, the lower byte into
// the lower half-word.
RPA_DEV u32x4 e4m3x8_to_bf16x8(const u32x2& w) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true))};
}

// float -> OCP E4M3 byte: the finite code nearest to x, ties to an even last
// mantissa bit; |x| is clamped to 448 (the largest finite code) first, NaN
// gives 0x7f, the sign of zero is kept.  Every step is exact: the exponent
// comes from the float's bits, the mantissa grid is a power-of-two scaling,
// and rintf rounds half to even.
RPA_DEV uint32_t f32_to_e4m3(float x) {
  const uint32_t bits = __builtin_bit_cast(uint32_t, x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  if ((bits & 0x7fffffffu) > 0x7f800000u) return 0x7fu;
  const float a = fminf(__builtin_fabsf(x), 448.f);
  if (a < 0.015625f) {   // below 2^-6: multiples of 2^-9; q = 8 is the smallest normal code 0x08
    return sign | static_cast<uint32_t>(rintf(a * 512.f));
  }
  const int e = static_cast<int>((__builtin_bit_cast(uint32_t, a) >> 23) & 0xffu) - 127;   // -6 .. 8
  uint32_t q = static_cast<uint32_t>(rintf(ldexpf(a, 3 - e)));                            // 8 .. 16
  int biased = e + 7;
  if (q == 16) {
    q = 8;
    ++biased;
  }
  return sign | (static_cast<uint32_t>(biased) << 3) | (q - 8);
}

// Eight bf16 (a 16-byte load) divided by `sc` in float32 and quantized to
// eight E4M3 bytes, element i in byte i.
RPA_DEV u32x2 bf16x8_to_e4m3x8(const u32x4& w, float sc) {
  uint32_t out[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = f32_to_e4m3(__builtin_bit_cast(float, w[j] << 16) / sc);
    const uint32_t hi = f32_to_e4m3(__builtin_bit_cast(float, w[j] & 0xffff0000u) / sc);
    out[j / 2] |= (lo | (hi << 8)) << (16 * (j % 2));
  }
  return u32x2{out[0], out[1]};
}

// Wave-uniform load through the constant address space, so it becomes a
// scalar load that does not wait behind the vector loads in flight.
typedef const int32_t __attribute__((address_space(4)))* const_i32_ptr;
RPA_DEV int32_t uniform_load(const int32_t* p, int idx) {
  return ((const_i32_ptr)(p))[idx];
}
typedef const float __attribute__((address_space(4)))* const_f32_ptr;
RPA_DEV float uniform_load(const float* p, int idx) {
  return ((const_f32_ptr)(p))[idx];
}

// KernelArgs: see rpa_kargs.h
//
// The pointers every work item needs first (its work item, the page table,
// Q, K and V) are separate kernel arguments ahead of the argument block, so
// that the build can preload them into scalar registers at wave launch
// (kernel-argument preloading, gfx950): the work-item load then needs no
// earlier load of the argument block, and the first K/V loads of a workgroup
// wait on two dependent memory round trips instead of three.
#define RPA_HOT_POINTERS                                                                  \
  const rpa_work_item* __restrict__ items, const int32_t* __restrict__ page_table,        \
      const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pages,               \
      const uint16_t* __restrict__ v_pages

RPA_DEV bool key_visible(int key, int pos, int kv_begin, int kv_end, int window) {
  return key >= kv_begin && key < kv_end && key <= pos && (window <= 0 || key > pos - window);
}
// The keys that key_visible() admits for position pos form one range
// [lo, lo + span]: key (>= 0) is visible iff unsigned(key - lo) <=
// unsigned(span).  An empty range is encoded as lo = -2^30, span = 0, which
// no key >= 0 passes.
RPA_DEV void visible_range(int pos, int kv_begin, int kv_end, int window, int& lo, int& span) {
  int a = kv_begin;
  if (window > 0 && pos - window + 1 > a) a = pos - window + 1;
  const int b = pos < kv_end - 1 ? pos : kv_end - 1;
  lo = b >= a ? a : -(1 << 30);
  span = b >= a ? b - a : 0;
}

// ---------------------------------------------------------------------------
// Prefill: NW waves x NB blocks of 32 query rows; BN keys per LDS tile;
// v_mfma_f32_32x32x16_bf16 for both products.
//
// K and V tiles go straight from HBM into LDS (buffer loads with an LDS
// destination: no staging registers), double buffered, in their natural
// [key][d] layout with a per-row XOR swizzle of the 16-byte chunks.
//
// S^T block (32 keys x 32 rows): lane (lq2 = lane/32, n = lane%32) holds keys
// 8b + 4*lq2 + t (b, t in 0..3) of row n in accumulator slot 4b + t.  The PV
// product consumes a 32-key block as two 16-key MFMAs h = 0, 1 whose k-slot
// 8*lq2 + i holds key 16h + 8*(i/4) + 4*lq2 + i%4 -- accumulator slots
// 8h .. 8h+7 of the same lane, so P never moves between lanes.  The V^T
// operand of those MFMAs is read with two transposing LDS reads
// (ds_read_b64_tr_b16): within a 16-lane group, lane i receives element i&3
// of the 8-byte chunk addressed by lane 4j + (i>>2) as its element j, so when
// lane L addresses key row r0 + (L>>2), columns d0 + 4*(L&3) .. +3, lane i
// gets keys r0 .. r0+3 of column d0 + i.
// ---------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef const void __attribute__((address_space(1)))* global_cptr;
typedef void __attribute__((address_space(3)))* lds_ptr;
typedef v4i16 __attribute__((address_space(3)))* lds_v4i16_ptr;

RPA_DEV f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16 bytes per lane from a buffer straight into LDS at dst + 16 * lane.
//
// Written as inline assembly on purpose: the compiler's own form of this load
// makes it assume that any later LDS read or barrier may depend on the copy,
// and it then drains every outstanding load (s_waitcnt vmcnt(0)) inside the
// tile loop, which defeats the multi-stage pipeline.  The kernels order these
// copies themselves: wait_tile_loads() on the issuing wave, then a barrier.
// The prefill prologue waits for every load (its own global loads and these
// copies) before the tile loop, and the loop issues no other vector loads, so
// a wait the compiler places for its own loads is never too short.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
RPA_DEV void buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, char* dst, int byte_off) {
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(dst)));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
               :: "v"(byte_off), "s"(base), "s"(rs) : "memory", "m0");
}
#pragma clang diagnostic pop
// A wave-uniform pointer / value kept in scalar registers (buffer
// descriptors must be built from them).
RPA_DEV const char* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v >> 32)));
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}
RPA_DEV uint32_t uniform_u32(uint32_t v) { return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v))); }
// 16 bytes per lane from a global address straight into LDS at dst + 16 * lane.
RPA_DEV void global_load_lds16(const char* src, char* dst) {
  __builtin_amdgcn_global_load_lds((global_cptr)(src), (lds_ptr)(dst), 16, 0, 0);
}
// Transposing 8-byte LDS read (see the layout note above).
RPA_DEV u32x2 lds_read_tr16(const char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(p)));
}

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, other counters left
// at their maxima).  Loads complete in issue order, so this waits for all but
// the N most recent.
template <int N>
RPA_DEV void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
RPA_DEV void wait_vmem() { wait_vmem_le<0>(); }

// Wait until the loads of the oldest staged tile are complete, given that
// `later` tiles of `LPT` loads each were staged after it.
template <int LPT, int MAXLATER>
RPA_DEV void wait_tile_loads(int later) {
  if constexpr (MAXLATER >= 3) {
    if (later >= 3) { wait_vmem_le<3 * LPT>(); return; }
  }
  if constexpr (MAXLATER >= 2) {
    if (later >= 2) { wait_vmem_le<2 * LPT>(); return; }
  }
  if constexpr (MAXLATER >= 1) {
    if (later >= 1) { wait_vmem_le<LPT>(); return; }
  }
  wait_vmem();
}

// DS = 2 splits the head dimension over a pair of waves: both waves of a pair
// hold the same 32 query rows, each the Q and O columns of one half of d; the
// two partial score blocks are added through LDS, so that each wave holds the
// full scores, runs the same softmax and accumulates its half of O.  This
// keeps Q and O of d = 512 within one wave's registers.
// Scheduling request for a block of N operand fetches of R LDS reads each,
// every fetch feeding M MFMAs: the first PF fetches are issued up front, then
// each fetch's MFMAs are followed by the reads of the fetch PF places later.
template <int N, int PF, int R, int M>
RPA_DEV void sched_reads_ahead() {
  __builtin_amdgcn_sched_group_barrier(0x100, PF * R, 0);   // DS reads
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, M, 0);      // MFMA
    if (i + PF < N) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  }
}

// Waves per SIMD a prefill shape is built for: two (fragments of up to 256
// VGPRs per wave), or three for a shape whose fragments fit 168 VGPRs.
template <int D, int BN, int NW, int NB, int NS, int DS>
struct PrefillWaves {
  static constexpr int PER_SIMD = 2;
};
template <>
struct PrefillWaves<128, 32, 4, 1, 2, 1> {
  static constexpr int PER_SIMD = 3;
};

template <int D, int BN, int NW, int NB, int NS, int DS = 1, bool KV8 = false>
struct PrefillCfg {
  static constexpr int NT = NW * 64;
  static constexpr int WAVES_PER_SIMD = PrefillWaves<D, BN, NW, NB, NS, DS>::PER_SIMD;
  static constexpr int DH = D / DS;                  // head columns per wave
  static constexpr int ROWS = (NW / DS) * NB * 32;   // query rows per workgroup
  static constexpr int ROW_B = D * 2;                // bytes per key row
  static constexpr int RPI = ROW_B >= 1024 ? 1 : 1024 / ROW_B;   // key rows per 1 KB block
  static constexpr int BLOCKS = BN * ROW_B / 1024;   // 1 KB blocks per K or V tile
  // LDS layout of a tile: 1 KB blocks (one direct load each) followed by a
  // pad; inside a block, row s sits at s*ROW_B with its 16-byte chunk c at
  // position c ^ x(s).  K and V use different pads / XORs, chosen so that the
  // operand reads hit distinct banks of the 64 x 4-byte LDS banks: a 16-byte
  // read serves 16 lanes per pass (K: 16 consecutive rows, one chunk), an
  // 8-byte transposing read 32 lanes (V: 4 consecutive rows x 64 bytes, which
  // must fall in the four distinct 64-byte bank windows of 256 bytes).  The
  // XOR touches bit 0 of the chunk for K; for V it touches bit 1, or with two
  // rows per block bit 2 (XV = 4: odd rows move to the neighbouring 64-byte
  // window, so a V read's offset depends on the parity of its 64-byte d block).
  static constexpr int PAD_K = RPI == 1 ? 16 : RPI == 2 ? 32 : 64;
  static constexpr int PAD_V = RPI == 2 ? 128 : 64;
  static constexpr int XV = RPI == 2 ? 4 : 2;       // chunk XOR of odd V rows
  static constexpr int BLK_K = 1024 + PAD_K;
  static constexpr int BLK_V = 1024 + PAD_V;
  static constexpr int TILE_K = BLOCKS * BLK_K;
  static constexpr int TILE_V = BLOCKS * BLK_V;
  static constexpr int STAGE_B = TILE_K + TILE_V;
  static constexpr int LOADS = BLOCKS / NW;          // 1 KB direct loads per wave per tensor
  // KV8 (an E4M3 cache): the NS stages in flight hold the tiles' bytes as
  // loaded (BN rows of D bytes, K then V), and CB tiles in the bf16 layout
  // above are converted from them inside the kernel: two when that still
  // lets a compute unit hold as many workgroups as the bf16 form (the next
  // tile is converted while the current one is used), else one (converted
  // after the current one's products).
  static constexpr int STAGE8 = 2 * BN * D;
  static constexpr int LOADS8 = BN * D / 1024 / NW;  // 1 KB direct loads per wave per tensor
  static constexpr int WGS = (160 * 1024) / (NS * STAGE_B) < 4 * WAVES_PER_SIMD * 64 / NT
                                 ? (160 * 1024) / (NS * STAGE_B)
                                 : 4 * WAVES_PER_SIMD * 64 / NT;   // bf16 form, per CU
  static constexpr int CB = 2 * STAGE_B + NS * STAGE8 <= (160 * 1024) / (WGS > 0 ? WGS : 1) ? 2 : 1;
  static constexpr int LDS_BYTES = KV8 ? CB * STAGE_B + NS * STAGE8 : NS * STAGE_B;
  static constexpr int LPT = 2 * (KV8 ? LOADS8 : LOADS);   // load instructions per wave per tile
  static_assert(NS >= 2 && NS <= 4, "2 to 4 stages");
  static_assert(!KV8 || (LOADS8 >= 1 && (BN * D) % (1024 * NW) == 0), "fp8 tile must split into 1 KB loads per wave");
  static_assert(!KV8 || (BN * D / 16) % NT == 0, "fp8 tile conversion: whole 16-byte pieces per thread");
  static_assert((NS - 2) * LPT < 64, "vmcnt field");
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(BLOCKS % NW == 0, "tile must split into 1 KB loads per wave");
  static_assert(16 % RPI == 0, "16-key steps must cover whole blocks");
  static_assert(DS == 1 || (DS == 2 && NW % 2 == 0 && BN == 32 && NB == 1), "d split: wave pairs, one 32x32 score block");
  // the score exchange of a d split reuses the K tile of the current stage
  static_assert(DS == 1 || NW * 4096 <= TILE_K, "score exchange must fit the K tile");
};

RPA_DEV int xor_k(int s) { return s & 1; }

template <int D, int BN, int NW, int NB, int NS, int DS, int SEG, bool KV8 = false, bool AP = false>
__global__ void __launch_bounds__(NW * 64, (PrefillWaves<D, BN, NW, NB, NS, DS>::PER_SIMD == 3 ? 3 : 1))
rpa_prefill_kernel(RPA_HOT_POINTERS, KernelArgs args) {
  using C = PrefillCfg<D, BN, NW, NB, NS, DS, KV8>;
  static_assert(!(AP && KV8), "new rows are taken from k_new / v_new with a bf16 cache only");
  // SEG: keys of an aligned run that lies in one page.  BN: a whole tile
  // (pages of a multiple of BN keys); BN / NW: the rows that one wave stages
  // of a tile; 0: a page id per lane.
  static_assert(SEG == 0 || SEG == BN || SEG * NW == BN, "page runs: a tile, a wave's rows of a tile, or none");
  constexpr bool UNI = SEG == BN;
  constexpr bool BUF = SEG > 0;   // buffer loads (no per-lane page lookups)
  constexpr int DH = C::DH;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  char* lds = reinterpret_cast<char*>(smem);

  const rpa_work_item it = items[blockIdx.x];
  // the work item's load goes out before the argument block's: nothing is
  // scheduled across this point, so the two loads are in flight together
  __builtin_amdgcn_sched_barrier(0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int rw = wave / DS;    // row block of this wave
  const int dh = wave % DS;    // head-column half of this wave (d split)
  const int n32 = lane & 31;   // MFMA column (query row) / A-operand row (key or d)
  const int lq2 = lane >> 5;   // lane half 0..1
  const int l16 = lane & 15;   // lane within a 16-lane group
  const int grp = lane >> 4;   // 16-lane group 0..3

  const int hq = args.num_q_heads;
  const int hkv = args.num_kv_heads;
  const int G = args.group;
  const int g = it.kv_head;
  const int32_t* __restrict__ pt_row = page_table + static_cast<int64_t>(it.seq) * args.max_pages;
  const uint16_t* __restrict__ kbase = k_pages;
  const uint16_t* __restrict__ vbase = v_pages;
  const int page_size = args.page_size;
  const int row_bytes = hkv * D * 2;   // bytes between consecutive key rows of a page
  const int row_bytes8 = hkv * D;      // the same for an E4M3 cache

  // Page ids of the key range, one per lane, 64 at a time (pw_ids holds pages
  // pw_base ..), loaded ahead of Q so that the first tile's staging does not
  // wait behind the Q loads.
  const int tile0 = (it.kv_begin / BN) * BN;  // tiles are aligned to BN keys
  const int wrap_pidx = tile0 / args.page_size;
  const int p_last = it.kv_end > tile0 ? (it.kv_end - 1) / args.page_size : -1;
  int pw_base = 0, pw_ids = 0;
  auto load_window = [&](int base) {
    pw_base = base;
    const int pi = base + lane;
    pw_ids = pi <= p_last ? pt_row[pi] : 0;
  };
  if (UNI) load_window(wrap_pidx);

  // ---- rows of this lane, Q fragments (B operand of S^T = K Q^T) ----
  int row_pos[NB];
  int vis_lo[NB], vis_span[NB];   // visible keys of the lane's rows (visible_range)
  u32x4 qf[NB][DH / 16];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r = (rw * NB + nb) * 32 + n32;
    const int tk = r / G;
    const int hh = r - tk * G;
    const bool row_ok = tk < it.q_count;
    row_pos[nb] = it.q_pos0 + tk;
    visible_range(row_pos[nb], it.kv_begin, it.kv_end, args.window, vis_lo[nb], vis_span[nb]);
    const int64_t row_off = (static_cast<int64_t>(it.q_start + tk) * hq + g * G + hh) * D;
#pragma unroll
    for (int kk = 0; kk < DH / 16; ++kk)
      qf[nb][kk] = row_ok ? load16(q + row_off + dh * DH + kk * 16 + lq2 * 8) : u32x4{0, 0, 0, 0};
  }
  // positions spanned by this wave's valid rows (tile skipping / mask-free tiles)
  const int tk_lo = (rw * NB * 32) / G;
  const int tk_hi_raw = ((rw + 1) * NB * 32 - 1) / G;
  const int tk_hi = tk_hi_raw < it.q_count - 1 ? tk_hi_raw : it.q_count - 1;
  const bool wave_active = tk_lo <= tk_hi;
  const int wpos_lo = it.q_pos0 + tk_lo;
  const int wpos_hi = it.q_pos0 + tk_hi;

  f32x16 o[DH / 32][NB];
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[db][nb] = f32x16{};
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = kNegInf;
    l_run[nb] = 0.f;
  }

  const int kv_begin = it.kv_begin;
  const int kv_end = it.kv_end;
  const int n_tiles = (kv_end - tile0 + BN - 1) / BN;
  // AP (an appending call): keys from the sequence's first new position
  // new0 on are this step's tokens, whose rows are k_new / v_new rows
  // new_row + key (the same row pitch as a page).  They are read from there:
  // their page slots are written by this launch, by the workgroup of each
  // query tile after its products, and read by none of its workgroups.
  // (An appending call passes its new rows to this launch only where every
  // item's new0 is a multiple of the buffer runs, SEG keys, so that no run
  // mixes pool and new rows: prefill_takes_new_rows.)
  [[maybe_unused]] const int new0 = AP ? it.new_pos0 : 0;
  [[maybe_unused]] const int64_t new_row = static_cast<int64_t>(it.q_start) - it.q_pos0;
  // Tile order: step t takes tile (t + rot) mod n_tiles of the range, with rot
  // chosen so that its global index (key / BN) is congruent to t modulo
  // n_tiles.  The online softmax is indifferent to the order of the tiles,
  // and neighbouring query tiles of a sliding window (same n_tiles, ranges
  // shifted by a few tiles) then read the same K/V tile at the same step: the
  // workgroups that one chiplet runs side by side fetch each tile from HBM
  // once and share it through their L2, instead of each streaming the window
  // in its own phase.  Full-causal ranges start at key 0 and keep their order.
  const int rot = n_tiles > 0 ? (n_tiles - (tile0 / BN) % n_tiles) % n_tiles : 0;
  auto key_of = [&](int t) {
    int u = t + rot;
    u -= u >= n_tiles ? n_tiles : 0;
    return tile0 + u * BN;
  };
  const int window = args.window;
  // An E4M3 cache: the K scale joins the score scale and the V scale the
  // output weight (both are per KV head, so they factor out of the products).
  float sl2 = args.scale_log2;
  float vsc = 1.f;
  if constexpr (KV8) {
    sl2 *= uniform_load(args.k_scales, g);
    vsc = uniform_load(args.v_scales, g);
  }

  // ---- the page of this wave's run of a tile (SEG = BN / NW) ----
  // Tiles are staged in order 0, 1, ..; each stage reads the page id the
  // previous one requested (a scalar load, one stage ahead).  The id is the
  // page of the run's first key inside the range, clipped to its last key,
  // so that only entries of the range are read.
  [[maybe_unused]] int run_page = 0, run_pidx = 0;
  auto fetch_run_page = [&](int ts) {
    int key = key_of(ts) + wave * SEG;
    key = key > kv_begin ? key : kv_begin;
    key = key < kv_end ? key : kv_end - 1;
    run_pidx = (key > 0 ? key : 0) / page_size;
    run_page = uniform_load(pt_row, run_pidx);
  };
  if constexpr (BUF && !UNI) {
    if (n_tiles > 0) fetch_run_page(0);
  }
  // The rows [lo, hi) of this wave's run of tile ts (k0 its first key): the
  // byte offset of the first in the pool, their byte count (0 for none) and
  // the bytes from the tile's first row to it.
  auto run_rows = [&](int ts, int k0, int lo, int hi, int rbytes, int esz, int64_t& base_off, uint32_t& nbytes,
                      int& rel_b) {
    const int64_t page = run_page;
    const int pidx = run_pidx;
    if (ts + 1 < n_tiles) fetch_run_page(ts + 1);
    const int s0 = k0 + wave * SEG;
    const int slo = s0 > lo ? s0 : lo;
    const int shi = s0 + SEG < hi ? s0 + SEG : hi;
    rel_b = (slo - k0) * rbytes;
    const int64_t off = ((page * page_size + (slo - pidx * page_size)) * hkv + g) * D * esz;
    const uint32_t n = shi > slo ? static_cast<uint32_t>((shi - slo - 1) * rbytes + D * esz) : 0u;
    // wave-uniform values: kept in scalar registers for the descriptors
    base_off = static_cast<int64_t>(
        (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(off >> 32)))) << 32) |
        static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(off))));
    nbytes = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(n)));
  };

  // ---- direct HBM -> LDS staging of one K/V tile ----
  // Load i of this wave fills block wave*LOADS + i of the K and V tiles; lane
  // l writes 16 bytes at +16*l of the block: key row s = 16*l / ROW_B of the
  // block, chunk position p, which holds source chunk p ^ x(s).
  int srow[C::LOADS], sgk[C::LOADS], sgv[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int blk = wave * C::LOADS + i;
    const int in_blk = lane * 16;
    const int sr = in_blk / C::ROW_B;
    const int p = (in_blk % C::ROW_B) / 16;
    srow[i] = blk * C::RPI + sr;
    sgk[i] = (p ^ xor_k(sr)) * 16;
    sgv[i] = (p ^ ((sr & 1) * C::XV)) * 16;
  }
  // Page and slot of the next tile to stage, advanced tile by tile (a tile
  // never crosses a page here) and reset when the order wraps to the start of
  // the range.  The range's page ids sit in a register, one per lane, 64 at a
  // time (pw_ids holds pages pw_base ..), so a stage reads its page id with
  // v_readlane instead of waiting on a load in the loop; a range of more than
  // 64 pages reloads the window, and waits for it, when the order leaves it.
  int st_u = rot;
  int st_pidx = 0, st_slot = 0, wrap_slot = 0;
  if constexpr (UNI) {
    wrap_slot = tile0 - wrap_pidx * page_size;
    const int kr = tile0 + rot * BN;
    st_pidx = kr / page_size;
    st_slot = kr - st_pidx * page_size;
  }

  // page slot row (page * page_size + slot) of the next tile's first key; advances
  auto next_tile_row = [&]() -> int64_t {
    if (static_cast<unsigned>(st_pidx - pw_base) >= 64u) {   // left the window (ranges of more than 64 pages)
      load_window(st_pidx);
      wait_vmem();
    }
    const int64_t page = __builtin_amdgcn_readlane(pw_ids, st_pidx - pw_base);
    const int64_t row = page * page_size + st_slot;
    st_slot += BN;
    if (st_slot == page_size) {
      st_slot = 0;
      ++st_pidx;
    }
    if (++st_u == n_tiles) {
      st_u = 0;
      st_pidx = wrap_pidx;
      st_slot = wrap_slot;
    }
    return row;
  };

  auto stage = [&](int ts, int buf) {
    const int k0 = key_of(ts);
    char* kdst = lds + buf * C::STAGE_B + wave * C::LOADS * C::BLK_K;
    char* vdst = lds + buf * C::STAGE_B + C::TILE_K + wave * C::LOADS * C::BLK_V;
    // Only keys [lo, hi) of the item's range are read: rows of the tile below
    // kv_begin (the first tile of a range that does not start on a tile
    // boundary) and past kv_end read as zero, and are masked later.
    const int lo = k0 > kv_begin ? k0 : kv_begin;
    const int hi = k0 + BN < kv_end ? k0 + BN : kv_end;
    if constexpr (UNI && !AP) {
      // The tile lies in one page.  The buffer starts at row lo and ends
      // after row hi - 1: rows below lo have negative offsets, which wrap
      // above the record count, so they read as zero like rows past hi.
      const int rel_b = (lo - k0) * row_bytes;
      const int64_t base_off = ((next_tile_row() + (lo - k0)) * hkv + g) * D;
      const uint32_t nbytes = static_cast<uint32_t>((hi - lo - 1) * row_bytes + D * 2);
      const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase + base_off, nbytes);
      const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase + base_off, nbytes);
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) {
        buffer_load_lds16(krs, kdst + i * C::BLK_K, srow[i] * row_bytes + sgk[i] - rel_b);
        buffer_load_lds16(vrs, vdst + i * C::BLK_V, srow[i] * row_bytes + sgv[i] - rel_b);
      }
    } else if constexpr (BUF && !AP) {
      // This wave's rows lie in one page: the same loads against a buffer
      // over the run's rows inside [lo, hi).
      int64_t base_off;
      uint32_t nbytes;
      int rel_b;
      run_rows(ts, k0, lo, hi, row_bytes, 2, base_off, nbytes, rel_b);
      const __amdgpu_buffer_rsrc_t krs = make_rsrc(reinterpret_cast<const char*>(kbase) + base_off, nbytes);
      const __amdgpu_buffer_rsrc_t vrs = make_rsrc(reinterpret_cast<const char*>(vbase) + base_off, nbytes);
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) {
        buffer_load_lds16(krs, kdst + i * C::BLK_K, srow[i] * row_bytes + sgk[i] - rel_b);
        buffer_load_lds16(vrs, vdst + i * C::BLK_V, srow[i] * row_bytes + sgv[i] - rel_b);
      }
    } else if constexpr (UNI) {
      // AP, the tile in one page: a tile below new0 reads the pool and one
      // from new0 on reads k_new / v_new, both as above (the same buffer
      // bounds).  No tile holds keys on both sides of new0 (new0 sits on a
      // tile boundary, see above).
      const int64_t trow = next_tile_row();   // page slot row of key k0
      const int rel_b = (lo - k0) * row_bytes;
      const uint32_t nbytes = uniform_u32(static_cast<uint32_t>((hi - lo - 1) * row_bytes + D * 2));
      const bool fresh = lo >= new0;
      const int64_t base_off = (((fresh ? new_row + lo : trow + (lo - k0))) * hkv + g) * D;
      const __amdgpu_buffer_rsrc_t krs = make_rsrc(uniform_ptr((fresh ? args.k_new : kbase) + base_off), nbytes);
      const __amdgpu_buffer_rsrc_t vrs = make_rsrc(uniform_ptr((fresh ? args.v_new : vbase) + base_off), nbytes);
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) {
        buffer_load_lds16(krs, kdst + i * C::BLK_K, srow[i] * row_bytes + sgk[i] - rel_b);
        buffer_load_lds16(vrs, vdst + i * C::BLK_V, srow[i] * row_bytes + sgv[i] - rel_b);
      }
    } else if constexpr (BUF) {
      // AP, this wave's rows in one page: the run's rows come from the pool,
      // or (from new0 on) from k_new / v_new.  No run holds keys on both
      // sides of new0 (new0 sits on a run boundary, see above).
      int64_t base_off;
      uint32_t nbytes;
      int rel_b;
      run_rows(ts, k0, lo, hi, row_bytes, 2, base_off, nbytes, rel_b);
      const int s0 = k0 + wave * SEG;
      const int slo = s0 > lo ? s0 : lo;
      const int shi = s0 + SEG < hi ? s0 + SEG : hi;
      const char* kb = reinterpret_cast<const char*>(kbase) + base_off;
      const char* vb = reinterpret_cast<const char*>(vbase) + base_off;
      if (slo >= new0 && shi > slo) {
        const int64_t noff = ((new_row + slo) * hkv + g) * D * 2;
        kb = reinterpret_cast<const char*>(args.k_new) + noff;
        vb = reinterpret_cast<const char*>(args.v_new) + noff;
      }
      const __amdgpu_buffer_rsrc_t krs = make_rsrc(uniform_ptr(kb), nbytes);
      const __amdgpu_buffer_rsrc_t vrs = make_rsrc(uniform_ptr(vb), nbytes);
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) {
        buffer_load_lds16(krs, kdst + i * C::BLK_K, srow[i] * row_bytes + sgk[i] - rel_b);
        buffer_load_lds16(vrs, vdst + i * C::BLK_V, srow[i] * row_bytes + sgv[i] - rel_b);
      }
    } else {
      // A wave's rows span pages: each lane looks up its row's page.  Rows
      // outside [lo, hi) are redirected to the nearest key of the range, so
      // every value read is a finite key of the range and no page before
      // kv_begin's is looked up.
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) {
        int key = k0 + srow[i];
        key = key < lo ? lo : (key < hi ? key : hi - 1);
        const bool fresh = AP && key >= new0;   // (AP) a new key: its k_new / v_new row
        const int pidx = key / page_size;
        const int64_t page = fresh ? 0 : pt_row[pidx];
        const int64_t row = fresh ? new_row + key : page * page_size + (key - pidx * page_size);
        const int64_t off = (row * hkv + g) * D * 2;
        global_load_lds16(reinterpret_cast<const char*>(fresh ? args.k_new : kbase) + off + sgk[i],
                          kdst + i * C::BLK_K);
        global_load_lds16(reinterpret_cast<const char*>(fresh ? args.v_new : vbase) + off + sgv[i],
                          vdst + i * C::BLK_V);
      }
    }
  };

  // ---- an E4M3 cache: direct HBM -> LDS loads of the tile's bytes ----
  // Load i of this wave fills 1 KB block wave*LOADS8 + i of the K and V bytes
  // (rows of D bytes, no XOR), with the same range rules as stage().
  auto stage8 = [&](int ts, int slot) {
    const int k0 = key_of(ts);
    char* kdst = lds + C::CB * C::STAGE_B + slot * C::STAGE8 + wave * C::LOADS8 * 1024;
    char* vdst = kdst + BN * D;
    const int lo = k0 > kv_begin ? k0 : kv_begin;
    const int hi = k0 + BN < kv_end ? k0 + BN : kv_end;
    const char* k8 = reinterpret_cast<const char*>(kbase);
    const char* v8 = reinterpret_cast<const char*>(vbase);
    if constexpr (UNI) {
      const int rel_b = (lo - k0) * row_bytes8;
      const int64_t base_off = ((next_tile_row() + (lo - k0)) * hkv + g) * D;
      const uint32_t nbytes = static_cast<uint32_t>((hi - lo - 1) * row_bytes8 + D);
      const __amdgpu_buffer_rsrc_t krs = make_rsrc(k8 + base_off, nbytes);
      const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v8 + base_off, nbytes);
#pragma unroll
      for (int i = 0; i < C::LOADS8; ++i) {
        const int at = (wave * C::LOADS8 + i) * 1024 + lane * 16;   // byte of the tile
        const int off = (at / D) * row_bytes8 + at % D - rel_b;
        buffer_load_lds16(krs, kdst + i * 1024, off);
        buffer_load_lds16(vrs, vdst + i * 1024, off);
      }
    } else if constexpr (BUF) {
      int64_t base_off;
      uint32_t nbytes;
      int rel_b;
      run_rows(ts, k0, lo, hi, row_bytes8, 1, base_off, nbytes, rel_b);
      const __amdgpu_buffer_rsrc_t krs = make_rsrc(k8 + base_off, nbytes);
      const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v8 + base_off, nbytes);
#pragma unroll
      for (int i = 0; i < C::LOADS8; ++i) {
        const int at = (wave * C::LOADS8 + i) * 1024 + lane * 16;   // byte of the tile
        const int off = (at / D) * row_bytes8 + at % D - rel_b;
        buffer_load_lds16(krs, kdst + i * 1024, off);
        buffer_load_lds16(vrs, vdst + i * 1024, off);
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::LOADS8; ++i) {
        const int at = (wave * C::LOADS8 + i) * 1024 + lane * 16;
        int key = k0 + at / D;
        key = key < lo ? lo : (key < hi ? key : hi - 1);
        const int pidx = key / page_size;
        const int64_t page = pt_row[pidx];
        const int64_t off = ((page * page_size + (key - pidx * page_size)) * hkv + g) * D + at % D;
        global_load_lds16(k8 + off, kdst + i * 1024);
        global_load_lds16(v8 + off, vdst + i * 1024);
      }
    }
  };
  // E4M3 bytes of stage `slot` -> bf16 tile `cb` in the layout the products
  // read (every E4M3 value is exact in bf16).  Thread t takes 16-byte pieces
  // t, t + NT, ...: 16 elements of one key row, i.e. two of its 16-byte bf16
  // chunks, each stored at its XOR position.
  auto convert = [&](int slot, int cb) {
    const char* src = lds + C::CB * C::STAGE_B + slot * C::STAGE8;
    char* dst = lds + cb * C::STAGE_B;
    // The piece offsets are recomputed at every call (a few VALU operations)
    // rather than kept in registers across the loop: held there, they leave
    // too few registers for the products' operand reads to run ahead.
    int me = tid;
    asm volatile("" : "+v"(me));
    // unrolled where the conversion runs before the products (few registers
    // live); rolled behind them, where unrolling spills (d = 512)
    constexpr int UNR = C::CB == 2 ? 8 : 1;
#pragma unroll UNR
    for (int tv = 0; tv < 2; ++tv) {   // K, then V
#pragma unroll UNR
      for (int j0 = 0; j0 < BN * D / 16; j0 += C::NT) {
        const int j = j0 + me;
        const int sr8 = (j * 16) / D;          // key row of the tile
        const int c = ((j * 16) % D) / 8;      // first bf16 chunk of the piece (even)
        const int sr = sr8 % C::RPI;
        const u32x4 x = *reinterpret_cast<const u32x4*>(src + tv * BN * D + j * 16);
        char* d = tv == 0 ? dst + (sr8 / C::RPI) * C::BLK_K + sr * C::ROW_B
                          : dst + C::TILE_K + (sr8 / C::RPI) * C::BLK_V + sr * C::ROW_B;
        const int xr = tv == 0 ? xor_k(sr) : (sr & 1) * C::XV;
        *reinterpret_cast<u32x4*>(d + (c ^ xr) * 16) = e4m3x8_to_bf16x8(u32x2{x[0], x[1]});
        *reinterpret_cast<u32x4*>(d + ((c + 1) ^ xr) * 16) = e4m3x8_to_bf16x8(u32x2{x[2], x[3]});
      }
    }
  };

  // per-lane LDS byte offsets of the MFMA operands (tile relative); the loop
  // counters only add immediates: kk*32 for K, 16-key steps and db*64 for V
  int kaddr[BN / 32];
#pragma unroll
  for (int kb = 0; kb < BN / 32; ++kb) {
    const int r = kb * 32 + n32;
    const int sr = r % C::RPI;
    kaddr[kb] = (r / C::RPI) * C::BLK_K + sr * C::ROW_B + (lq2 ^ xor_k(sr)) * 16;
  }
  // vaddr[half][par]: V reads of the 64-byte d blocks of parity par (the odd
  // rows' XOR on chunk bit 2 maps d block b to b ^ 1, i.e. +64 or -64 bytes)
  int vaddr[2][2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int r = 4 * lq2 + (l16 >> 2) + 8 * half;
    const int sr = r % C::RPI;
    const int cl = 2 * (grp & 1) + ((l16 & 3) >> 1);
    const int xv = (sr & 1) * C::XV;
    const int base = C::TILE_K + (r / C::RPI) * C::BLK_V + sr * C::ROW_B + (l16 & 1) * 8;
    if constexpr (C::XV == 4) {
      vaddr[half][0] = base + cl * 16 + (xv ? 64 : 0);
      vaddr[half][1] = base + cl * 16 - (xv ? 64 : 0);
    } else {
      vaddr[half][0] = vaddr[half][1] = base + (cl ^ xv) * 16;
    }
  }

  // tile starting at key kt fully masked for this wave's rows: nothing to add
  auto tile_skipped = [&](int kt) {
    return !wave_active || kt > wpos_hi || kt + BN <= kv_begin || (window > 0 && kt + BN - 1 <= wpos_lo - window);
  };
  // ---- S^T = K Q^T for the K tile at kbuf ----
  // LDS reads run KPF operands ahead of the MFMAs that use them, so that the
  // read latency overlaps the matrix work instead of stalling every MFMA.
  auto scores = [&](const char* kbuf, f32x16 (&acc)[BN / 32][NB]) {
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[kb][nb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < DH / 16; ++kk) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kbuf + kaddr[kb] + dh * DH * 2 + kk * 32);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[kb][nb] = mfma32(a, qf[nb][kk], acc[kb][nb]);
      }
    }
    constexpr int KREADS = (DH / 16) * (BN / 32);
    constexpr int KPF = KREADS < 4 ? KREADS : 4;
    sched_reads_ahead<KREADS, KPF, 1, NB>();
  };

  // ---- mask + online softmax of the tile at keys k0.. -> bf16 probabilities pf ----
  auto softmax = [&](f32x16 (&sc)[BN / 32][NB], int k0, u32x4 (&pf)[BN / 16][NB]) __attribute__((always_inline)) {
    // Scores stay raw; scale*log2(e) is folded into one FMA per element.
    // The running maximum m_run is only raised when a row's new maximum
    // exceeds it by more than 8 (in log2 units), so O is rescaled rarely;
    // every p stays below 2^8 and the result is unchanged because the same
    // reference maximum enters both O and l.
    const bool full = (k0 >= kv_begin) && (k0 + BN <= kv_end) && (k0 + BN - 1 <= wpos_lo) &&
                      (window <= 0 || k0 > wpos_hi - window);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (!full) {
        // key - lo for element j of block kb is rel + kb*32 + 8*(j/4) + (j%4)
        const int rel = k0 + 4 * lq2 - vis_lo[nb];
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const uint32_t d = static_cast<uint32_t>(rel + kb * 32 + 8 * (j >> 2) + (j & 3));
            if (d > static_cast<uint32_t>(vis_span[nb])) sc[kb][nb][j] = kNegInf;
          }
      }
      // Maximum over this lane's keys; a row's keys are split over lanes n and
      // n + 32.  A row's maximum exceeds m_run + 8 iff one of its halves does,
      // so the exchange of the halves' maxima is only needed on the (rare)
      // path that raises m_run.
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sc[kb][nb][j]);
      if (__any(mx * sl2 > m_run[nb] + 8.f)) {
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mx2 = mx * sl2;   // the row's tile maximum in log2 units (scale > 0)
        const float m_new = fmaxf(m_run[nb], mx2);
        // 0 when the row had no visible key yet; 1 for a row that still has none
        const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run[nb] - m_new);
        m_run[nb] = m_new;
        l_run[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < DH / 32; ++db) o[db][nb] *= alpha;
      }
      const float base = (m_run[nb] == kNegInf) ? 0.f : m_run[nb];
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float p[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            p[i] = fast_exp2(__builtin_fmaf(sc[kb][nb][8 * h + i], sl2, -base));
            lsum += p[i];
          }
          pf[kb * 2 + h][nb] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                     pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
        }
      }
      l_run[nb] += lsum;
    }
  };

  // ---- O^T += V^T P^T for the V tile at ks: V^T operands by two transposing reads each ----
  // The V^T operands are read PF products ahead of the MFMA that uses them (a
  // rolling window of PF operands in registers), the order pinned with
  // scheduling barriers: left to itself, the scheduler issues each operand's
  // reads right before its MFMA, which then waits a whole LDS round trip
  // (measured: 4-9 % of the prefill kernel's time).
  auto pv = [&](const u32x4 (&pf)[BN / 16][NB], const char* ks) __attribute__((always_inline)) {
    constexpr int VOPS = (BN / 16) * (DH / 32);
    constexpr int PF = VOPS < 4 ? VOPS : 4;
    auto vread = [&](int i) {
      const int ks16 = i / (DH / 32);
      const int db = i % (DH / 32);
      const char* vrow = ks + ks16 * (16 / C::RPI) * C::BLK_V;
      const u32x2 l2 = lds_read_tr16(vrow + vaddr[0][db & 1] + dh * DH * 2 + db * 64);
      const u32x2 h2 = lds_read_tr16(vrow + vaddr[1][db & 1] + dh * DH * 2 + db * 64);
      return u32x4{l2[0], l2[1], h2[0], h2[1]};
    };
    u32x4 win[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) win[i] = vread(i);
#pragma unroll
    for (int i = 0; i < VOPS; ++i) {
      const int ks16 = i / (DH / 32);
      const int db = i % (DH / 32);
      const u32x4 a = win[i % PF];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[db][nb] = mfma32(a, pf[ks16][nb], o[db][nb]);
      if (i + PF < VOPS) win[i % PF] = vread(i + PF);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- the products of tile `tile`, whose K/V tile is at ks ----
  auto products = [&](int tile, char* ks) __attribute__((always_inline)) {
    const int k0 = key_of(tile);
    const bool skip = tile_skipped(k0);
    f32x16 sc[BN / 32][NB];
    if (!skip) scores(ks, sc);
    if constexpr (DS == 2) {
      // ---- d split: add the partner wave's partial scores ----
      // Every wave has finished its reads of this K tile, whose space then
      // carries the exchange (16 B per lane and store, lanes contiguous).
      // Float addition commutes, so both waves of a pair hold identical sums.
      __syncthreads();
      f32x4* xb = reinterpret_cast<f32x4*>(ks);
      if (!skip) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          xb[(wave * 4 + c) * 64 + lane] = f32x4{sc[0][0][4 * c], sc[0][0][4 * c + 1], sc[0][0][4 * c + 2], sc[0][0][4 * c + 3]};
      }
      __syncthreads();
      if (!skip) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const f32x4 y = xb[((wave ^ 1) * 4 + c) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[0][0][4 * c + e] += y[e];
        }
      }
    }
    if (!skip) {
      u32x4 pf[BN / 16][NB];
      softmax(sc, k0, pf);
      pv(pf, ks);
    }
  };

  if constexpr (!KV8) {
    // NS-stage pipeline: while tile t is used, the loads of tiles t+1 ..
    // t+NS-1 are in flight; one barrier per tile guards the reuse of a buffer.
    // (Measured: two tiles per barrier step, or running half of the waves one
    // phase behind the other half, are both slower on this kernel.)
#pragma unroll
    for (int t = 0; t < NS - 1; ++t)
      if (t < n_tiles) stage(t, t);
    if constexpr (BUF) {
      // Q and the first tiles: every load of the prologue is complete before the loop
      wait_vmem();
    } else {
      // the first tile must have landed
      const int later = (n_tiles < NS - 1 ? n_tiles : NS - 1) - 1;
      wait_tile_loads<C::LPT, NS - 2>(later < 0 ? 0 : later);
    }
    __syncthreads();

    for (int tile = 0; tile < n_tiles; ++tile) {
      const int ts = tile + NS - 1;   // into the buffer of tile - 1, released by the last barrier
      if (ts < n_tiles) stage(ts, ts % NS);
      products(tile, lds + (tile % NS) * C::STAGE_B);
      // the next tile must have landed; later ones may still be in flight
      {
        const int staged_last = (tile + NS - 1 < n_tiles ? tile + NS - 1 : n_tiles - 1);
        const int later = staged_last - (tile + 1);
        wait_tile_loads<C::LPT, NS - 2>(later < 0 ? 0 : later);
      }
      __syncthreads();
    }
  } else {
    // An E4M3 cache: NS stages of loaded bytes and CB converted bf16 tiles.
    // At the barrier that opens step t, bf16 tile t is complete and stage t
    // has been converted, so step t loads tile t+NS into it.  With two bf16
    // tiles, step t converts tile t+1 (landed before that barrier) into the
    // tile that t-1 used, before the products of tile t; with one, it
    // converts tile t+1 after them, behind a second barrier.
    for (int t = 0; t < NS; ++t)
      if (t < n_tiles) stage8(t, t);
    if constexpr (BUF) {
      // Q and the first tiles: every load of the prologue is complete before the loop
      wait_vmem();
    } else {
      const int later = (n_tiles < NS ? n_tiles : NS) - 1;   // tiles staged after tile 0
      wait_tile_loads<C::LPT, NS - 1>(later < 0 ? 0 : later);
    }
    __syncthreads();
    if (n_tiles > 0) convert(0, 0);
    if constexpr (C::CB == 2) {
      const int later = (n_tiles < NS ? n_tiles : NS) - 2;   // tiles staged after tile 1
      wait_tile_loads<C::LPT, NS - 1>(later < 0 ? 0 : later);
    }
    __syncthreads();

    for (int tile = 0; tile < n_tiles; ++tile) {
      if (tile + NS < n_tiles) stage8(tile + NS, tile % NS);
      const int staged_last = tile + NS < n_tiles ? tile + NS : n_tiles - 1;
      if constexpr (C::CB == 2) {
        if (tile + 1 < n_tiles) convert((tile + 1) % NS, (tile + 1) & 1);
        products(tile, lds + (tile & 1) * C::STAGE_B);
        // the bytes of tile + 2 must have landed; later ones may be in flight
        const int later = staged_last - (tile + 2);
        wait_tile_loads<C::LPT, NS - 1>(later < 0 ? 0 : later);
      } else {
        products(tile, lds);
        const int later = staged_last - (tile + 1);   // tile + 1 must have landed
        wait_tile_loads<C::LPT, NS - 1>(later < 0 ? 0 : later);
        __syncthreads();   // every wave is done with the bf16 tile
        if (tile + 1 < n_tiles) convert((tile + 1) % NS, 0);
      }
      __syncthreads();
    }
  }

  // AP: split 0 of a query tile writes its tokens' K/V rows (KV head g)
  // into their page slots after its products (the copy kernel's work for
  // these tokens): 16-byte pieces, U of them per thread in flight (more
  // spill registers at d = 256 and 512).
  auto write_new_rows = [&]() {
    if constexpr (AP) {
      if (it.self_append == 0) return;
      constexpr int CH = D / 8;   // 16-byte pieces per row
      constexpr int U = 8;
      const int n = it.q_count * CH * 2;   // (token, K or V, piece)
      uint16_t* kpool = const_cast<uint16_t*>(kbase);
      uint16_t* vpool = const_cast<uint16_t*>(vbase);
      for (int i0 = tid; i0 < n; i0 += C::NT * U) {
        u32x4 val[U];
        int64_t dst[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int idx = i0 + u * C::NT;
          const bool ok = idx < n;
          const int rr = idx / CH;
          const int c = idx - rr * CH;
          const int r = rr >> 1;
          const int pos = it.q_pos0 + r;
          const int64_t page = ok ? pt_row[pos / page_size] : 0;
          const int64_t src = (static_cast<int64_t>(it.q_start + r) * hkv + g) * D + c * 8;
          val[u] = ok ? load16(((rr & 1) ? args.v_new : args.k_new) + src) : u32x4{0, 0, 0, 0};
          dst[u] = ((page * page_size + pos % page_size) * hkv + g) * D + c * 8;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int idx = i0 + u * C::NT;
          if (idx < n) *reinterpret_cast<u32x4*>((((idx / CH) & 1) ? vpool : kpool) + dst[u]) = val[u];
        }
      }
    }
  };

  constexpr int OROWS = NB * 32;   // rows per wave
  if (it.split_group >= 0) {
    // ---- a split of a long item: normalised fp32 O and base-2 LSE per row ----
    // Row r of split i sits at row i * ROWS of the group's partial block; the
    // merge kernel that follows the launch merges the block (the same
    // arithmetic as the decode splits' merge).
    const int64_t prow = static_cast<int64_t>(it.partial_base) * 16 + static_cast<int64_t>(it.split_index) * C::ROWS;
    float inv[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float l = l_run[nb] + __shfl_xor(l_run[nb], 32);
      inv[nb] = l > 0.f ? vsc / l : 0.f;
      const float base = (m_run[nb] == kNegInf) ? 0.f : m_run[nb];
      const int r = (rw * NB + nb) * 32 + n32;
      if (lq2 == 0 && dh == 0 && r / G < it.q_count)
        args.partial_lse[prow + r] = l > 0.f ? base + __builtin_log2f(l) : kNegInf;
    }
    // The fp32 rows go through LDS, in SP passes of CW columns, so that the
    // stores write whole rows (16 contiguous bytes per lane, lanes along a
    // row), as the bf16 epilogue does; the 16-byte row pad keeps the 16-byte
    // LDS writes of 16 rows on distinct banks.  Tiles whose LDS cannot hold a
    // 32-column pass store from registers instead.
    constexpr int SP = (DH % 32 == 0 && NW * OROWS * (DH * 4 + 16) <= C::LDS_BYTES) ? 1
                     : (DH % 64 == 0 && NW * OROWS * (DH * 2 + 16) <= C::LDS_BYTES) ? 2
                     : (DH % 128 == 0 && NW * OROWS * (DH + 16) <= C::LDS_BYTES) ? 4 : 0;
    if constexpr (SP > 0) {
      constexpr int CW = DH / SP;          // columns per pass
      constexpr int RP = CW * 4 + 16;      // LDS bytes per staged row
      constexpr int CPF = CW * 4 / 16;     // 16-byte chunks per row per pass
      constexpr int RPF = 64 / CPF;        // rows per store instruction
      static_assert(CPF <= 64 && 64 % CPF == 0 && OROWS % RPF == 0, "whole rows per store");
      char* fst = lds + wave * OROWS * RP;
      const int fr = lane / CPF;
      const int fc = lane - fr * CPF;
#pragma unroll
      for (int ps = 0; ps < SP; ++ps) {
        if (ps > 0) __syncthreads();   // the previous pass's reads are done
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int db = ps * (CW / 32); db < (ps + 1) * (CW / 32); ++db)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const float* v = reinterpret_cast<const float*>(&o[db][nb]) + 4 * b;
              *reinterpret_cast<f32x4*>(fst + (nb * 32 + n32) * RP + ((db - ps * (CW / 32)) * 32 + 8 * b + 4 * lq2) * 4) =
                  f32x4{v[0] * inv[nb], v[1] * inv[nb], v[2] * inv[nb], v[3] * inv[nb]};
            }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < OROWS / RPF; ++i) {
          const int lr = i * RPF + fr;
          const int r = rw * NB * 32 + lr;
          const f32x4 v = *reinterpret_cast<const f32x4*>(fst + lr * RP + fc * 16);
          if (r / G < it.q_count)
            *reinterpret_cast<f32x4*>(args.partial_o + (prow + r) * D + dh * DH + ps * CW + fc * 4) = v;
        }
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int r = (rw * NB + nb) * 32 + n32;
        if (r / G < it.q_count) {
          float* dst = args.partial_o + (prow + r) * D + dh * DH + lq2 * 4;
#pragma unroll
          for (int db = 0; db < DH / 32; ++db)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const float* v = reinterpret_cast<const float*>(&o[db][nb]) + 4 * b;
              *reinterpret_cast<f32x4*>(dst + db * 32 + b * 8) =
                  f32x4{v[0] * inv[nb], v[1] * inv[nb], v[2] * inv[nb], v[3] * inv[nb]};
            }
        }
      }
    }
    write_new_rows();
    return;
  }

  // ---- epilogue: O / l -> bf16, staged through LDS ----
  // A lane holds d = 32*db + 8*b + 4*lq2 + t of row n32, i.e. 8-byte pieces
  // strewn over 32 rows; stored directly, every store instruction would touch
  // 32 lines with 16 bytes each, and with all workgroups of a launch ending
  // together those partial-line writes queue at the L2 for microseconds.  So
  // each wave first writes its rows into its own LDS slice (the K/V buffers
  // are free after the loop's last barrier), then stores 16 contiguous bytes
  // per lane with consecutive lanes along a row: whole rows per instruction.
  // The row pitch OP (8 bytes of pad) keeps the 8-byte LDS writes of 32 rows
  // on distinct banks.
  constexpr int OP = DH * 2 + 8;
  constexpr int CPR = DH * 2 / 16;   // 16-byte chunks per row slice
  constexpr int RPS = 64 / CPR;      // rows per store instruction
  static_assert(NW * OROWS * OP <= C::LDS_BYTES, "output staging must fit the tile buffers");
  static_assert(64 % CPR == 0 && OROWS % RPS == 0, "whole rows per store");
  char* ost = lds + wave * OROWS * OP;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float l = l_run[nb] + __shfl_xor(l_run[nb], 32);
    const float inv = l > 0.f ? vsc / l : 0.f;
    char* srow = ost + (nb * 32 + n32) * OP + lq2 * 8;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float* v = reinterpret_cast<const float*>(&o[db][nb]) + 4 * b;
        *reinterpret_cast<u32x2*>(srow + (db * 32 + b * 8) * 2) =
            u32x2{pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv)};
      }
    }
  }
  __syncthreads();
  const int cr = lane / CPR;
  const int cc = lane - cr * CPR;
#pragma unroll
  for (int i = 0; i < OROWS / RPS; ++i) {
    const int lr = i * RPS + cr;          // nb * 32 + n of the wave's rows
    const int r = rw * NB * 32 + lr;      // row of the workgroup's tile
    const int tk = r / G;
    const int hh = r - tk * G;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ost + lr * OP + cc * 16);
    if (tk < it.q_count)
      *reinterpret_cast<u32x4*>(args.out + (static_cast<int64_t>(it.q_start + tk) * hq + g * G + hh) * D +
                                dh * DH + cc * 8) = v;
  }
  write_new_rows();
}

// ---------------------------------------------------------------------------
// Split merge: out = sum_i 2^(lse_i - M) O_i / sum_i 2^(lse_i - M), M = max_i lse_i.
// One workgroup per group; each thread owns one 4-float column of one row,
// with enough threads (MergeCfg::THREADS) that a decode group's 16 x D/4 columns
// take at most two passes and each thread's loads are in flight together.
// ---------------------------------------------------------------------------
template <int D>
struct MergeCfg {
  static constexpr int THREADS = 4 * D < 1024 ? 4 * D : 1024;
};
// Merges the n partials of one split group (rows q_count * G of tokens from
// q_start, KV head kv_head) into the bf16 output; threads tid of nthreads.
// Split i's rows start at row i * rps of the group's block (rps = 16 for
// decode splits, the tile's row count for prefill splits).  Each thread
// takes PER column slots per pass (tid, tid + nthreads, ...) and issues the
// loads of all of them before it combines any, so a group of up to
// PER * nthreads slots costs one memory round trip; the arithmetic of a
// slot does not depend on PER.
template <int D, int PER = 1>
RPA_DEV void merge_group(const KernelArgs& args, int q_start, int q_count, int kv_head, int partial_base,
                         int n, int rps, int tid, int nthreads) {
  constexpr int C4 = D / 4;
  constexpr int NB = 8;   // splits fetched per batch: every load of a batch is in flight at once
  const int rows = q_count * args.group;
  const int total = rows * C4;
  // Device-scope loads (they miss the compute unit's vector cache and read
  // what other compute units wrote): the fused merge runs in the launch
  // that writes the partials, after the last split's ticket, and a cached
  // line of the workspace may predate its other splits' stores.
  constexpr int kDeviceScope = 16;   // the cache-policy bit of a device-scope load
  const __amdgpu_buffer_rsrc_t lrs =
      make_rsrc(args.partial_lse + static_cast<int64_t>(partial_base) * 16, static_cast<uint32_t>(n * rps * 4));
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(args.partial_o + static_cast<int64_t>(partial_base) * 16 * D,
                                               static_cast<uint32_t>(n * rps * D * 4));
  for (int i0 = tid; i0 < total; i0 += nthreads * PER) {
    float mx[PER], wsum[PER];
    f32x4 acc[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      mx[p] = kNegInf;
      wsum[p] = 0.f;
      acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int s0 = 0; s0 < n; s0 += NB) {
      float l[PER][NB];
      f32x4 v[PER][NB];
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int idx = i0 + p * nthreads;
        const int r = idx / C4;
        const int c = idx - r * C4;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const bool ok = s0 + b < n && idx < total;
          const int slot_row = (s0 + b) * rps + r;
          l[p][b] = ok ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lrs, slot_row * 4, 0,
                                                                                        kDeviceScope))
                       : kNegInf;
          v[p][b] = ok ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       ors, (slot_row * D + c * 4) * 4, 0, kDeviceScope))
                       : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        float bm = mx[p];
#pragma unroll
        for (int b = 0; b < NB; ++b) bm = fmaxf(bm, l[p][b]);
        const float base = (bm == kNegInf) ? 0.f : bm;
        const float rescale = fast_exp2(mx[p] - base);   // running sums to the new maximum
        wsum[p] *= rescale;
        acc[p] *= rescale;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float w = fast_exp2(l[p][b] - base);
          wsum[p] += w;
          acc[p] += w * v[p][b];
        }
        mx[p] = bm;
      }
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int idx = i0 + p * nthreads;
      if (idx >= total) break;
      const int r = idx / C4;
      const int c = idx - r * C4;
      const f32x4 o = acc[p] * (wsum[p] > 0.f ? 1.f / wsum[p] : 0.f);
      const int tk = r / args.group;
      const int hh = r - tk * args.group;
      uint16_t* dst = args.out + (static_cast<int64_t>(q_start + tk) * args.num_q_heads +
                                  kv_head * args.group + hh) * D + c * 4;
      *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
  }
}

// Workgroup (x, y) merges column slots y * THREADS .. of group x: a prefill
// group's 128-256 rows are spread over several workgroups (one round of
// loads each) instead of being walked by one.
template <int D>
__global__ void __launch_bounds__(MergeCfg<D>::THREADS) rpa_merge_kernel(KernelArgs args) {
  const rpa_work_item grp = args.groups[blockIdx.x];
  // rows per split: a prefill tile's, 16 for a decode item, 32 for a two-block one
  merge_group<D>(args, grp.q_start, grp.q_count, grp.kv_head, grp.partial_base, grp.num_splits,
                 grp.kind == 0 ? args.prefill_rows : grp.kind == 2 ? 32 : 16, blockIdx.y * blockDim.x + threadIdx.x,
                 blockDim.x * gridDim.y);
}

// ---------------------------------------------------------------------------
// Decode: rows = q_count * G <= 16 * RB; NW waves take 32-key chunks round
// robin.  Every wave issues all loads of a chunk before touching any of them;
// the waves are combined in a fixed order through LDS (bitwise reproducible).
// RB = 2 holds two blocks of 16 rows (a single token of 32 grouped heads, or
// a few tokens of a smaller group) over the same K/V fragments: each key
// row loaded serves twice the rows, and such items stay off the prefill
// kernel, whose 128-256-row tiles they would leave mostly empty.
// ---------------------------------------------------------------------------
template <int D, int NW, int RB = 1>
struct DecodeCfg {
  static constexpr int NT = NW * 64;
  static constexpr int ROWS = 16 * RB;                // query rows of an item
  static constexpr int NCH = D / 8;                   // 16-byte chunks per key row
  static constexpr int NU = (NCH + 15) / 16;          // V chunk rounds per lane
  static constexpr int OSTRIDE = D + 4;               // floats per LDS row (padded)
  static constexpr int LDS_O = (NW / 2) * ROWS * OSTRIDE; // tree-combine slots
  static constexpr int LDS_BYTES = LDS_O * 4 + NW * ROWS * 2 * 4 + 16;   // + merge flag
};

// Second launch bound: waves per SIMD to fit (two, so a compute unit holds two
// workgroups of 4 waves; one for D = 512 whose fragments need the full file,
// and for two row blocks at D = 256).
// KV8: the pools hold OCP FP8 E4M3 bytes with one K and one V scale per KV
// head; each lane loads 8 bytes where the bf16 form loads 16 and converts
// them to the same bf16 operand layout.  The K scale joins the score scale
// and the V scale the output weight (both are per KV head, so they factor
// out of the dot products).
// AP: an appending call (the fused KV write of the items holding all of
// their sequence's new tokens); a separate instantiation, so that plain calls
// carry none of its code.
template <int D, int NW, int SEG, bool KV8, int RB = 1, bool AP = false>
__global__ void __launch_bounds__(NW * 64, (D >= 512 || (RB == 2 && D >= 256)) ? 1 : 2)
rpa_decode_kernel(RPA_HOT_POINTERS, KernelArgs args) {
  using C = DecodeCfg<D, NW, RB>;
  constexpr int ROWS = C::ROWS;
  // Column chunks (8 columns) of V and O: MFMA row m of pass u holds chunk
  // u*16 + m, or with an E4M3 cache of two or more passes (V16) chunk
  // m*NU + u, so that a lane's chunks are contiguous bytes, loaded 16 at a time.
  constexpr bool V16 = KV8 && C::NU >= 2;
  static_assert(!V16 || C::NU * 16 == C::NCH, "every lane holds NU chunks");
  auto vchunk = [](int u, int m) { return V16 ? m * C::NU + u : u * 16 + m; };
  extern __shared__ __attribute__((aligned(16))) float dsm[];
  float* lds_o = dsm;                     // [NW/2][ROWS][OSTRIDE]
  float* lds_m = dsm + C::LDS_O;          // [NW][ROWS]
  float* lds_l = lds_m + NW * ROWS;       // [NW][ROWS]
  int* lds_flag = reinterpret_cast<int*>(lds_l + NW * ROWS);

  const rpa_work_item it = items[blockIdx.x];
  // the work item's load goes out before the argument block's: nothing is
  // scheduled across this point, so the two loads are in flight together
  __builtin_amdgcn_sched_barrier(0);
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
  const int32_t* __restrict__ pt_row = page_table + static_cast<int64_t>(it.seq) * args.max_pages;
  using KVT = typename std::conditional<KV8, uint8_t, uint16_t>::type;
  constexpr int ESZ = sizeof(KVT);
  const KVT* __restrict__ kbase = reinterpret_cast<const KVT*>(k_pages);
  const KVT* __restrict__ vbase = reinterpret_cast<const KVT*>(v_pages);
  const int page_size = args.page_size;
  const int64_t row_stride = static_cast<int64_t>(hkv) * D;
  const int kv_begin = it.kv_begin;
  const int kv_end = it.kv_end;
  const int window = args.window;
  float sl2 = args.scale_log2;
  float vscale = 1.f;
  if constexpr (KV8) {
    sl2 *= uniform_load(args.k_scales, g);
    vscale = uniform_load(args.v_scales, g);
  }

  // query row n = rb*16 + ln: token n / G, head n % G
  int pos[RB];
  bool row_ok[RB];
  u32x4 qf[RB][D / 32];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = rb * 16 + ln;
    const int tk = r / G;
    const int hh = r - tk * G;
    row_ok[rb] = r < rows;
    pos[rb] = it.q_pos0 + tk;
    const int64_t q_off = (static_cast<int64_t>(it.q_start + tk) * hq + g * G + hh) * D;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      // An E4M3 cache: lane lq reads 16 contiguous key bytes per pair of
      // 32-column slices (columns 64p + 16lq ..), so the Q columns of slot kk
      // are those bytes' half kk % 2 (the score sums over the columns, so one
      // permutation applied to both operands leaves it unchanged).
      const int dq = KV8 ? (kk >> 1) * 64 + lq * 16 + (kk & 1) * 8 : kk * 32 + lq * 8;
      qf[rb][kk] = row_ok[rb] ? load16(q + q_off + dq) : u32x4{0, 0, 0, 0};
    }
  }

  f32x4 o[RB][C::NU][8];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int u = 0; u < C::NU; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[rb][u][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = kNegInf;
    l_run[rb] = 0.f;
  }

  // 32-key chunks aligned to 32 keys.  SEG > 0: each aligned run of SEG keys
  // of a chunk (the whole chunk, or each 16-key half) lies in one page, whose
  // id the wave reads one chunk ahead (the page of the run's first key inside
  // the item's range, clipped to its last key, so that only entries of the
  // range are read).  SEG = 0 (page sizes that are not a multiple of 16
  // keys): a page id per lane.
  constexpr int NSEG = SEG > 0 ? 32 / SEG : 1;
  const int chunk0 = (kv_begin / 32) * 32;
  const int n_chunks = (kv_end - chunk0 + 31) / 32;
  const int row_bytes = static_cast<int>(row_stride) * ESZ;   // bytes between key rows of a page
  int next_page[NSEG];
  auto fetch_pages = [&](int k0) {
#pragma unroll
    for (int sg = 0; sg < NSEG; ++sg) {
      int key = k0 + sg * SEG > kv_begin ? k0 + sg * SEG : kv_begin;
      key = key < kv_end ? key : kv_end - 1;
      next_page[sg] = uniform_load(pt_row, (key > 0 ? key : 0) / page_size);
    }
  };
  auto first_page = [&]() {
    if constexpr (SEG > 0) {
      if (wave < n_chunks) fetch_pages(chunk0 + wave * 32);
    }
  };

  // ---- fused KV write (appending calls, AP) ----
  // An item that holds every new token of its sequence writes the new K/V
  // rows whose keys lie in its key range into their page slots itself (the
  // new tokens are the last keys of the sequence, so one split of a group
  // holds each): the rows go through HBM once and no other launch is needed.
  // Each new key's rows are written by the wave that takes the key's chunk,
  // before that wave loads the chunk, so the wave reads them back from the
  // pages in its own program order (a wave-scope release and acquire, no
  // barrier): the loop below is the same as for a call without new rows,
  // and the other waves start their loads without waiting.  With an fp8
  // cache the rows are quantized on the way, and the chunk load converts the
  // stored bytes as it does every other key's.  A lane's first row piece is
  // requested before the first chunk's page id, so that the two wait on one
  // memory round trip rather than two.
  if constexpr (AP) {
    int new_lo = 0, n_new = 0;
    if (it.self_append != 0) {
      new_lo = it.q_pos0 > kv_begin ? it.q_pos0 : kv_begin;
      const int new_hi = it.q_pos0 + it.q_count < kv_end ? it.q_pos0 + it.q_count : kv_end;
      n_new = new_hi > new_lo ? new_hi - new_lo : 0;
    }
    constexpr int CH = D / 8;   // 16-byte pieces of a bf16 row
    const int pieces = 2 * n_new * CH;
    // piece i: the K (i < n_new*CH) or V row of key new_lo + r, piece c
    auto piece = [&](int i, int& which, int& key, int& c) {
      which = i >= n_new * CH;
      const int rem = i - which * n_new * CH;
      const int r = rem / CH;
      c = rem - r * CH;
      key = new_lo + r;
    };
    auto mine = [&](int key) { return ((key - chunk0) / 32) % NW == wave; };
    auto src_of = [&](int key, int c) {
      return (static_cast<int64_t>(it.q_start + (key - it.q_pos0)) * hkv + g) * D + c * 8;
    };
    u32x4 x0 = u32x4{0, 0, 0, 0};
    int page0 = 0;
    bool first = false;
    if (lane < pieces) {
      int which, key, c;
      piece(lane, which, key, c);
      first = mine(key);
      if (first) {
        x0 = load16((which ? args.v_new : args.k_new) + src_of(key, c));
        page0 = pt_row[key / page_size];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    first_page();
    __builtin_amdgcn_sched_barrier(0);
    for (int i = lane; i < pieces; i += 64) {
      int which, key, c;
      piece(i, which, key, c);
      if (!mine(key)) continue;
      u32x4 x = x0;
      int page = page0;
      if (i != lane || !first) {
        x = load16((which ? args.v_new : args.k_new) + src_of(key, c));
        page = pt_row[key / page_size];
      }
      const int64_t slot =
          ((static_cast<int64_t>(page) * page_size + (key - (key / page_size) * page_size)) * hkv + g) * D + c * 8;
      if constexpr (KV8) {
        uint8_t* pool = const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(which ? v_pages : k_pages));
        *reinterpret_cast<u32x2*>(pool + slot) = bf16x8_to_e4m3x8(x, which ? args.v_scales[g] : args.k_scales[g]);
      } else {
        uint16_t* pool = const_cast<uint16_t*>(which ? v_pages : k_pages);
        *reinterpret_cast<u32x4*>(pool + slot) = x;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    first_page();
  }

  for (int ch = wave; ch < n_chunks; ch += NW) {
    const int k0 = chunk0 + ch * 32;
    // keys of this lane: K rows k0 + 16*kb + ln; V rows k0 + 4*lq + j and k0 + 16 + 4*lq + j
    u32x4 kf[2][D / 32];
    u32x4 vf[C::NU][8];
    // KV8: the raw bytes of kf (16 per lane and column pair, see qf) and
    // of vf (with V16, lane ln holds column chunks ln * NU .. ln * NU + NU - 1,
    // two per 16-byte load; else chunk ln)
    [[maybe_unused]] u32x4 kr[2][D / 64 > 0 ? D / 64 : 1];
    [[maybe_unused]] u32x2 vr[C::NU][8];
    [[maybe_unused]] u32x4 vr2[C::NU / 2 > 0 ? C::NU / 2 : 1][8];
    if constexpr (SEG > 0) {
      // Buffer loads against each run's valid key rows [lo, hi); rows outside
      // read as zero (negative offsets wrap above the record count, an empty
      // run has no records), so there are no branches and no NaN reads.
      int page[NSEG];
#pragma unroll
      for (int sg = 0; sg < NSEG; ++sg) page[sg] = next_page[sg];
      if (ch + NW < n_chunks) fetch_pages(k0 + NW * 32);
      __amdgpu_buffer_rsrc_t krs[NSEG], vrs[NSEG];
      int rel[NSEG];   // run start - lo (<= 0)
#pragma unroll
      for (int sg = 0; sg < NSEG; ++sg) {
        const int s0 = k0 + sg * SEG;
        const int lo = s0 > kv_begin ? s0 : kv_begin;
        const int hi = s0 + SEG < kv_end ? s0 + SEG : kv_end;
        const int64_t lo_off =
            ((static_cast<int64_t>(page[sg]) * page_size + (lo - (lo / page_size) * page_size)) * hkv + g) * D;
        const uint32_t nbytes = hi > lo ? static_cast<uint32_t>((hi - lo - 1) * row_bytes + D * ESZ) : 0u;
        krs[sg] = make_rsrc(kbase + lo_off, nbytes);
        vrs[sg] = make_rsrc(vbase + lo_off, nbytes);
        rel[sg] = s0 - lo;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int sg = (kb * 16) / (SEG > 0 ? SEG : 32);
        const int off = (rel[sg] + kb * 16 - sg * SEG + ln) * row_bytes + lq * 8 * ESZ;
        if constexpr (KV8) {
#pragma unroll
          for (int p = 0; p < D / 64; ++p) kr[kb][p] = buffer_load16(krs[sg], off + lq * 8 + p * 64);
        } else {
#pragma unroll
          for (int kk = 0; kk < D / 32; ++kk) kf[kb][kk] = buffer_load16(krs[sg], off + kk * 64);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int sg = (j < 4 ? 0 : 16) / (SEG > 0 ? SEG : 32);
        const int key_rel = rel[sg] - sg * SEG + ((j < 4) ? (lq * 4 + j) : (16 + lq * 4 + j - 4));
        if constexpr (V16) {
#pragma unroll
          for (int u2 = 0; u2 < C::NU / 2; ++u2)
            vr2[u2][j] = buffer_load16(vrs[sg], key_rel * row_bytes + (ln * C::NU + 2 * u2) * 8);
        } else {
#pragma unroll
          for (int u = 0; u < C::NU; ++u) {
            const int c = u * 16 + ln;
            if constexpr (KV8) vr[u][j] = c < C::NCH ? buffer_load8(vrs[sg], key_rel * row_bytes + c * 8) : u32x2{0, 0};
            else vf[u][j] = c < C::NCH ? buffer_load16(vrs[sg], key_rel * row_bytes + c * 16) : u32x4{0, 0, 0, 0};
          }
        }
      }
    } else {
      int kkey[2], vkey[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kkey[kb] = k0 + kb * 16 + ln;
#pragma unroll
      for (int j = 0; j < 8; ++j) vkey[j] = k0 + ((j < 4) ? (lq * 4 + j) : (16 + lq * 4 + j - 4));
      int kpid[2] = {0, 0}, vpid[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      // every page id first, then the K/V loads
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kkey[kb] >= kv_begin && kkey[kb] < kv_end) kpid[kb] = pt_row[kkey[kb] / page_size];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (vkey[j] >= kv_begin && vkey[j] < kv_end) vpid[j] = pt_row[vkey[j] / page_size];
      auto kv_row = [&](int key, int pid) -> int64_t {
        const int slot = key - (key / page_size) * page_size;
        return ((static_cast<int64_t>(pid) * page_size + slot) * hkv + g) * D;
      };
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bool ok = kkey[kb] >= kv_begin && kkey[kb] < kv_end;
        const int64_t off = kv_row(kkey[kb], kpid[kb]);
        if constexpr (KV8) {
#pragma unroll
          for (int p = 0; p < D / 64; ++p) kr[kb][p] = ok ? load16b(kbase + off + p * 64 + lq * 16) : u32x4{0, 0, 0, 0};
        } else {
#pragma unroll
          for (int kk = 0; kk < D / 32; ++kk) kf[kb][kk] = ok ? load16(kbase + off + kk * 32 + lq * 8) : u32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool ok = vkey[j] >= kv_begin && vkey[j] < kv_end;
        const int64_t off = kv_row(vkey[j], vpid[j]);
        if constexpr (V16) {
#pragma unroll
          for (int u2 = 0; u2 < C::NU / 2; ++u2)
            vr2[u2][j] = ok ? load16b(vbase + off + (ln * C::NU + 2 * u2) * 8) : u32x4{0, 0, 0, 0};
        } else {
#pragma unroll
          for (int u = 0; u < C::NU; ++u) {
            const int c = u * 16 + ln;
            if constexpr (KV8) vr[u][j] = (ok && c < C::NCH) ? load8(vbase + off + c * 8) : u32x2{0, 0};
            else vf[u][j] = (ok && c < C::NCH) ? load16(vbase + off + c * 8) : u32x4{0, 0, 0, 0};
          }
        }
      }
    }
    if constexpr (KV8) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int p = 0; p < D / 64; ++p) {
          kf[kb][2 * p] = e4m3x8_to_bf16x8(u32x2{kr[kb][p][0], kr[kb][p][1]});
          kf[kb][2 * p + 1] = e4m3x8_to_bf16x8(u32x2{kr[kb][p][2], kr[kb][p][3]});
        }
      if constexpr (V16) {
#pragma unroll
        for (int u2 = 0; u2 < C::NU / 2; ++u2)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            vf[2 * u2][j] = e4m3x8_to_bf16x8(u32x2{vr2[u2][j][0], vr2[u2][j][1]});
            vf[2 * u2 + 1][j] = e4m3x8_to_bf16x8(u32x2{vr2[u2][j][2], vr2[u2][j][3]});
          }
      } else {
#pragma unroll
        for (int u = 0; u < C::NU; ++u)
#pragma unroll
          for (int j = 0; j < 8; ++j) vf[u][j] = e4m3x8_to_bf16x8(vr[u][j]);
      }
    }
    u32x4 pf[RB];
    float alpha[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) s[kb] = mfma16(kf[kb][kk], qf[rb][kk], s[kb]);
      }
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = k0 + kb * 16 + lq * 4 + j;
          float x = s[kb][j] * sl2;
          if (!key_visible(key, pos[rb], kv_begin, kv_end, window)) x = kNegInf;
          s[kb][j] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = xor_max(mx);
      const float m_new = fmaxf(m_run[rb], mx);
      const float base = (m_new == kNegInf) ? 0.f : m_new;
      alpha[rb] = fast_exp2(m_run[rb] - base);
      m_run[rb] = m_new;
      float p[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = fast_exp2(s[0][j] - base);
        p[4 + j] = fast_exp2(s[1][j] - base);
      }
      float lsum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) lsum += p[j];
      l_run[rb] = l_run[rb] * alpha[rb] + lsum;
      pf[rb] = u32x4{pack_bf16x2_split(p[0], p[1]), pack_bf16x2_split(p[2], p[3]),
                     pack_bf16x2_split(p[4], p[5]), pack_bf16x2_split(p[6], p[7])};
    }
#pragma unroll
    for (int u = 0; u < C::NU; ++u) {
      u32x4 vt[8];
      transpose8x8(vf[u], vt);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[rb][u][e] = mfma16(vt[e], pf[rb], o[rb][u][e] * alpha[rb]);
    }
  }

  // ---- combine the waves: common max, per-wave weight, fixed-order tree ----
  float lsum[RB], base[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_wave = xor_sum(l_run[rb]);
    if (lq == 0) {
      lds_m[wave * ROWS + rb * 16 + ln] = m_run[rb];
      lds_l[wave * ROWS + rb * 16 + ln] = l_wave;
    }
  }
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = rb * 16 + ln;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, lds_m[w * ROWS + r]);
    base[rb] = (mx == kNegInf) ? 0.f : mx;
    lsum[rb] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) lsum[rb] += fast_exp2(lds_m[w * ROWS + r] - base[rb]) * lds_l[w * ROWS + r];
    const float inv = lsum[rb] > 0.f ? 1.f / lsum[rb] : 0.f;
    const float wscale = fast_exp2(m_run[rb] - base[rb]) * inv * vscale;   // this wave's share, normalised
#pragma unroll
    for (int u = 0; u < C::NU; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[rb][u][e] *= wscale;
  }
  // lane (lq, ln) holds O[row rb*16 + ln][d = 8*chunk(u, 4lq + j) + e]; slot rows are padded by 4 floats
  auto slot_ptr = [&](int slot, int rb, int u, int j) {
    return reinterpret_cast<f32x4*>(lds_o + (slot * ROWS + rb * 16 + ln) * C::OSTRIDE + vchunk(u, lq * 4 + j) * 8);
  };
#pragma unroll
  for (int half = NW / 2; half >= 1; half /= 2) {
    if (wave >= half && wave < 2 * half) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (!row_ok[rb]) continue;
#pragma unroll
        for (int u = 0; u < C::NU; ++u)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (vchunk(u, lq * 4 + j) < C::NCH) {
              f32x4* dst = slot_ptr(wave - half, rb, u, j);
              dst[0] = f32x4{o[rb][u][0][j], o[rb][u][1][j], o[rb][u][2][j], o[rb][u][3][j]};
              dst[1] = f32x4{o[rb][u][4][j], o[rb][u][5][j], o[rb][u][6][j], o[rb][u][7][j]};
            }
      }
    }
    __syncthreads();
    if (wave < half) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (!row_ok[rb]) continue;
#pragma unroll
        for (int u = 0; u < C::NU; ++u)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (vchunk(u, lq * 4 + j) < C::NCH) {
              const f32x4* src = slot_ptr(wave, rb, u, j);
              const f32x4 lo = src[0], hi = src[1];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                o[rb][u][e][j] += lo[e];
                o[rb][u][4 + e][j] += hi[e];
              }
            }
      }
    }
    if (half > 1) __syncthreads();
  }
  // ---- output rows (or the split's partial) through LDS, whole rows per store ----
  // Wave 0 holds the combined rows; it writes them into slot 0 of the tree
  // (row-major, rows padded to OSTRIDE floats) and every thread then stores
  // 16 contiguous bytes of a row, consecutive threads along the row, instead
  // of wave 0 storing 16-byte pieces strewn over 16 rows.
  if (wave == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (!row_ok[rb]) continue;
#pragma unroll
      for (int u = 0; u < C::NU; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (vchunk(u, lq * 4 + j) < C::NCH) {
            f32x4* dst = slot_ptr(0, rb, u, j);
            dst[0] = f32x4{o[rb][u][0][j], o[rb][u][1][j], o[rb][u][2][j], o[rb][u][3][j]};
            dst[1] = f32x4{o[rb][u][4][j], o[rb][u][5][j], o[rb][u][6][j], o[rb][u][7][j]};
          }
    }
  }
  __syncthreads();
  const bool split = it.split_group >= 0;
  constexpr int C4 = D / 4;
  if (!split) {
    for (int idx = tid; idx < rows * C4; idx += C::NT) {
      const int r = idx / C4;
      const int c = idx - r * C4;
      const f32x4 v = *reinterpret_cast<const f32x4*>(lds_o + r * C::OSTRIDE + c * 4);
      const int rt = r / G;
      const int rh = r - rt * G;
      *reinterpret_cast<u32x2*>(args.out + (static_cast<int64_t>(it.q_start + rt) * hq + g * G + rh) * D + c * 4) =
          u32x2{pack_bf16x2_split(v[0], v[1]), pack_bf16x2_split(v[2], v[3])};
    }
    return;
  }
  // a split's rows take RB consecutive 16-row partial slots
  const int64_t slot = static_cast<int64_t>(it.partial_base) + static_cast<int64_t>(it.split_index) * RB;
  for (int idx = tid; idx < rows * C4; idx += C::NT) {
    const int r = idx / C4;
    const int c = idx - r * C4;
    *reinterpret_cast<f32x4*>(args.partial_o + (slot * 16 + r) * D + c * 4) =
        *reinterpret_cast<const f32x4*>(lds_o + r * C::OSTRIDE + c * 4);
  }
  if (wave == 0 && lq == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      if (row_ok[rb])
        args.partial_lse[slot * 16 + rb * 16 + ln] = (lsum[rb] > 0.f) ? base[rb] + __builtin_log2f(lsum[rb]) : kNegInf;
  }
  if (!args.fused_merge) return;

  // ---- last split of the group merges it (the group's ticket counts arrivals) ----
  // The workspace is uncached device memory: the stores above reach memory,
  // where every workgroup's loads and the ticket atomic see them, once each
  // wave's vmcnt reaches zero.  The split that draws the last ticket then
  // reads all partials back (its own included) and merges them in split order
  // with the same arithmetic as the merge kernel, and resets the ticket for
  // the next call.  Those reads are device-scope loads (merge_group), which
  // miss this compute unit's vector cache: it may hold a line of the
  // workspace read earlier in the launch by another group's merge on this
  // unit (16 LSEs of a slot are 64 bytes, so two groups' slots share a
  // 128-byte line), from before this group's splits wrote it.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    *lds_flag = __hip_atomic_fetch_add(args.merge_tickets + it.split_group, 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT) == it.num_splits - 1;
  __syncthreads();
  if (*lds_flag == 0) return;
  asm volatile("" ::: "memory");   // no read of the workspace moves above the ticket
  // column slots per thread: a group of 8 rows (16 at d <= 128) in one pass of four waves
  constexpr int MPER = D >= 512 ? 4 : D >= 128 ? 2 : 1;
  merge_group<D, MPER>(args, it.q_start, it.q_count, it.kv_head, it.partial_base, it.num_splits, ROWS, tid, C::NT);
  if (tid == 0) __hip_atomic_store(args.merge_tickets + it.split_group, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// KV append: the step's new keys and values into their pages, before the
// attention kernels read them (the pages' kernel writes the new tokens' K/V
// into the cache within the attention call: "TPU Deep Dive", chapter 8).
// The new token at flattened index t of sequence s is at position
// kv_len_s - q_len_s + (t - cu_q_lens[s]); its row of KV head g goes to slot
// pos % page_size of page page_table[s][pos / page_size].  One workgroup per
// work item; the items whose split index is 0 cover every (token, KV head)
// pair of the step exactly once, and each copies its tokens' rows of its KV
// head with 16-byte loads and stores, consecutive threads along a row.
// ---------------------------------------------------------------------------
constexpr int kAppendThreads = 256;

// KV8: the pools hold E4M3 bytes; each new element is divided by its KV
// head's scale and quantized (f32_to_e4m3), 8 bytes written per 16 read.
template <int D, bool KV8>
__global__ void __launch_bounds__(kAppendThreads)
rpa_append_kernel(const rpa_work_item* __restrict__ items, const int32_t* __restrict__ page_table,
                  const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
                  uint16_t* __restrict__ k_dst, uint16_t* __restrict__ v_dst, KernelArgs args) {
  const rpa_work_item it = items[blockIdx.x];
  // decode items that hold all of their sequence's new tokens write them
  // themselves (the decode kernel's fused write), and so do prefill items
  // when the prefill launch takes the call's new rows (prefill_writes)
  if (it.split_index != 0 || (it.self_append != 0 && (it.kind != 0 || args.prefill_writes != 0))) return;
  constexpr int CH = D / 8;   // 16-byte chunks per row
  const int hkv = args.num_kv_heads;
  const int ps = args.page_size;
  const int32_t* pt_row = page_table + static_cast<int64_t>(it.seq) * args.max_pages;
  const int n = it.q_count * CH;
  for (int i = threadIdx.x; i < n; i += kAppendThreads) {
    const int r = i / CH;
    const int c = i - r * CH;
    const int pos = it.q_pos0 + r;
    const int64_t page = pt_row[pos / ps];
    const int64_t src = (static_cast<int64_t>(it.q_start + r) * hkv + it.kv_head) * D + c * 8;
    const int64_t dst = ((page * ps + pos % ps) * hkv + it.kv_head) * D + c * 8;
    if constexpr (KV8) {
      const float ks = args.k_scales[it.kv_head];
      const float vs = args.v_scales[it.kv_head];
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(k_dst) + dst) =
          bf16x8_to_e4m3x8(*reinterpret_cast<const u32x4*>(k_new + src), ks);
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(v_dst) + dst) =
          bf16x8_to_e4m3x8(*reinterpret_cast<const u32x4*>(v_new + src), vs);
    } else {
      *reinterpret_cast<u32x4*>(k_dst + dst) = *reinterpret_cast<const u32x4*>(k_new + src);
      *reinterpret_cast<u32x4*>(v_dst + dst) = *reinterpret_cast<const u32x4*>(v_new + src);
    }
  }
}

// ---------------------------------------------------------------------------
// fp8 staging: the pages of the sequences that the prefill kernel serves in an
// fp8 call, converted to bf16 (E4M3 value times the KV head's scale, rounded
// to nearest even) into pages of a bf16 pool, which the prefill kernel then
// reads through the pool's own page table.  Workgroup (b, y) converts part y
// of staged page b (kStageChunks 16-byte chunks per part, so that a launch
// has enough workgroups when pages are large); stage[3b .. 3b+2] =
// (sequence, page of the sequence, page of the pool).  Each thread converts
// 16 bytes at a time (one KV head's row segment, as D is a multiple of 16)
// into 32 bytes.
// ---------------------------------------------------------------------------
constexpr int kStageThreads = 256;
constexpr int kStageChunks = 4 * kStageThreads;

RPA_DEV uint32_t scale_bf16x2(uint32_t w, float sc) {
  const float lo = __builtin_bit_cast(float, w << 16);
  const float hi = __builtin_bit_cast(float, w & 0xffff0000u);
  return pack_bf16x2(lo * sc, hi * sc);
}

template <int D>
__global__ void __launch_bounds__(kStageThreads)
rpa_stage_kernel(const int32_t* __restrict__ stage, const int32_t* __restrict__ page_table,
                 const uint8_t* __restrict__ k8, const uint8_t* __restrict__ v8, uint16_t* __restrict__ k_dst,
                 uint16_t* __restrict__ v_dst, KernelArgs args) {
  const int seq = stage[blockIdx.x * 3];
  const int lp = stage[blockIdx.x * 3 + 1];
  const int slot = stage[blockIdx.x * 3 + 2];
  const int hkv = args.num_kv_heads;
  const int64_t page_elems = static_cast<int64_t>(args.page_size) * hkv * D;
  const int64_t src = static_cast<int64_t>(page_table[static_cast<int64_t>(seq) * args.max_pages + lp]) * page_elems;
  const int64_t dst = static_cast<int64_t>(slot) * page_elems;
  const int n16 = static_cast<int>(page_elems / 16);
  const int first = blockIdx.y * kStageChunks;
  const int last = first + kStageChunks < n16 ? first + kStageChunks : n16;
  for (int i = first + threadIdx.x; i < last; i += kStageThreads) {
    const int g = ((i * 16) / D) % hkv;
    const float ks = args.k_scales[g];
    const float vs = args.v_scales[g];
    const u32x4 kr = *reinterpret_cast<const u32x4*>(k8 + src + i * 16);
    const u32x4 vr = *reinterpret_cast<const u32x4*>(v8 + src + i * 16);
    const u32x4 ka = e4m3x8_to_bf16x8(u32x2{kr[0], kr[1]});
    const u32x4 kb = e4m3x8_to_bf16x8(u32x2{kr[2], kr[3]});
    const u32x4 va = e4m3x8_to_bf16x8(u32x2{vr[0], vr[1]});
    const u32x4 vb = e4m3x8_to_bf16x8(u32x2{vr[2], vr[3]});
    u32x4* kd = reinterpret_cast<u32x4*>(k_dst + dst + i * 16);
    u32x4* vd = reinterpret_cast<u32x4*>(v_dst + dst + i * 16);
    kd[0] = u32x4{scale_bf16x2(ka[0], ks), scale_bf16x2(ka[1], ks), scale_bf16x2(ka[2], ks), scale_bf16x2(ka[3], ks)};
    kd[1] = u32x4{scale_bf16x2(kb[0], ks), scale_bf16x2(kb[1], ks), scale_bf16x2(kb[2], ks), scale_bf16x2(kb[3], ks)};
    vd[0] = u32x4{scale_bf16x2(va[0], vs), scale_bf16x2(va[1], vs), scale_bf16x2(va[2], vs), scale_bf16x2(va[3], vs)};
    vd[1] = u32x4{scale_bf16x2(vb[0], vs), scale_bf16x2(vb[1], vs), scale_bf16x2(vb[2], vs), scale_bf16x2(vb[3], vs)};
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int D, int BN, int NW, int NB, int NS, int DS, int SEG, bool KV8, bool AP>
static hipError_t launch_prefill_v(const KernelArgs& a, int n_items, hipStream_t stream) {
  using C = PrefillCfg<D, BN, NW, NB, NS, DS, KV8>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&rpa_prefill_kernel<D, BN, NW, NB, NS, DS, SEG, KV8, AP>),
        hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((rpa_prefill_kernel<D, BN, NW, NB, NS, DS, SEG, KV8, AP>), dim3(n_items), dim3(C::NT),
                     C::LDS_BYTES, stream, a.items, a.page_table, a.q, a.k, a.v, a);
  return hipGetLastError();
}

// bf16 pages with new rows given (an appending call): the AP form, which
// reads the new tokens' keys from them and writes their rows.
template <int D, int BN, int NW, int NB, int NS, int DS, int SEG, bool KV8>
static hipError_t launch_prefill_u(const KernelArgs& a, int n_items, hipStream_t stream) {
  if constexpr (!KV8) {
    if (a.k_new != nullptr) return launch_prefill_v<D, BN, NW, NB, NS, DS, SEG, false, true>(a, n_items, stream);
  }
  return launch_prefill_v<D, BN, NW, NB, NS, DS, SEG, KV8, false>(a, n_items, stream);
}

// Keys of a run that the prefill launch of this shape loads through one
// buffer descriptor: a tile (BN) or a wave's rows of it (BN / NW) when pages
// hold whole runs and the offsets fit 32 bits; 0: each lane looks up its
// row's page.  esz: bytes per cache element.
template <int D, int BN, int NW, int NB, int NS, int DS>
static int prefill_run_keys(const KernelArgs& a, int esz) {
  constexpr int WR = BN / NW;
  const bool fits = int64_t(a.page_size) * a.num_kv_heads * D * esz < (int64_t(1) << 31);
  return !fits ? 0 : a.page_size % BN == 0 ? BN : a.page_size % WR == 0 ? WR : 0;
}

// WITH_KV8 = false builds a shape for bf16 pages only (kv8 must be false).
template <int D, int BN, int NW, int NB, int NS, int DS, bool WITH_KV8 = true>
static hipError_t launch_prefill_t(const KernelArgs& a, int n_items, bool kv8, hipStream_t stream) {
  constexpr int WR = BN / NW;
  const int seg = prefill_run_keys<D, BN, NW, NB, NS, DS>(a, kv8 ? 1 : 2);
  if constexpr (WITH_KV8) {
    if (kv8) {
      if (seg == BN) return launch_prefill_u<D, BN, NW, NB, NS, DS, BN, true>(a, n_items, stream);
      if (seg == WR) return launch_prefill_u<D, BN, NW, NB, NS, DS, WR, true>(a, n_items, stream);
      return launch_prefill_u<D, BN, NW, NB, NS, DS, 0, true>(a, n_items, stream);
    }
  } else {
    if (kv8) return hipErrorInvalidValue;
  }
  if (seg == BN) return launch_prefill_u<D, BN, NW, NB, NS, DS, BN, false>(a, n_items, stream);
  if (seg == WR) return launch_prefill_u<D, BN, NW, NB, NS, DS, WR, false>(a, n_items, stream);
  return launch_prefill_u<D, BN, NW, NB, NS, DS, 0, false>(a, n_items, stream);
}

template <int D, int NW, int SEG, bool KV8, int RB, bool AP>
static hipError_t launch_decode_v(const KernelArgs& a, int n_items, hipStream_t stream) {
  using C = DecodeCfg<D, NW, RB>;
  if constexpr (C::LDS_BYTES > 64 * 1024) {   // beyond the default dynamic LDS limit
    static bool attr_set = false;
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&rpa_decode_kernel<D, NW, SEG, KV8, RB, AP>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
  }
  hipLaunchKernelGGL((rpa_decode_kernel<D, NW, SEG, KV8, RB, AP>), dim3(n_items), dim3(C::NT), C::LDS_BYTES, stream,
                     a.items, a.page_table, a.q, a.k, a.v, a);
  return hipGetLastError();
}

// Appending calls (new rows given) run the AP form, with four waves.
template <int D, int NW, bool KV8 = false, int RB = 1>
static hipError_t launch_decode_u(const KernelArgs& a, int n_items, hipStream_t stream) {
  const bool ap = a.k_new != nullptr;
  if (a.page_size % 32 == 0)
    return ap ? launch_decode_v<D, 4, 32, KV8, RB, true>(a, n_items, stream)
              : launch_decode_v<D, NW, 32, KV8, RB, false>(a, n_items, stream);
  if (a.page_size % 16 == 0)
    return ap ? launch_decode_v<D, 4, 16, KV8, RB, true>(a, n_items, stream)
              : launch_decode_v<D, NW, 16, KV8, RB, false>(a, n_items, stream);
  return ap ? launch_decode_v<D, 4, 0, KV8, RB, true>(a, n_items, stream)
            : launch_decode_v<D, NW, 0, KV8, RB, false>(a, n_items, stream);
}

// Eight-wave workgroups are not used for D = 512: two waves per SIMD cannot
// hold its fragments.  The fp8 form and the two-block (32-row) form are built
// with four waves only; there is no two-block form for D = 512.
template <int D>
static hipError_t launch_decode_t(const KernelArgs& a, int n_items, int waves, bool kv8, int rows,
                                  hipStream_t stream) {
  if constexpr (D < 512) {
    if (rows > 16) {
      if (kv8) return launch_decode_u<D, 4, true, 2>(a, n_items, stream);
      return launch_decode_u<D, 4, false, 2>(a, n_items, stream);
    }
  } else {
    if (rows > 16) return hipErrorInvalidValue;
  }
  if (kv8) return launch_decode_u<D, 4, true>(a, n_items, stream);
  if constexpr (D < 512) {
    if (waves == 8) return launch_decode_u<D, 8>(a, n_items, stream);
  }
  return launch_decode_u<D, 4>(a, n_items, stream);
}

template <int D>
static hipError_t launch_append_t(const KernelArgs& a, int n_items, const void* k_new, const void* v_new,
                                  void* k_dst, void* v_dst, bool kv8, hipStream_t stream) {
  if (kv8)
    hipLaunchKernelGGL((rpa_append_kernel<D, true>), dim3(n_items), dim3(kAppendThreads), 0, stream, a.items,
                       a.page_table, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       static_cast<uint16_t*>(k_dst), static_cast<uint16_t*>(v_dst), a);
  else
    hipLaunchKernelGGL((rpa_append_kernel<D, false>), dim3(n_items), dim3(kAppendThreads), 0, stream, a.items,
                       a.page_table, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       static_cast<uint16_t*>(k_dst), static_cast<uint16_t*>(v_dst), a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_stage_t(const KernelArgs& a, const int32_t* stage, int n_pages, void* k_dst, void* v_dst,
                                 hipStream_t stream) {
  const int64_t n16 = int64_t(a.page_size) * a.num_kv_heads * D / 16;
  const int parts = static_cast<int>((n16 + kStageChunks - 1) / kStageChunks);
  hipLaunchKernelGGL((rpa_stage_kernel<D>), dim3(n_pages, parts), dim3(kStageThreads), 0, stream, stage, a.page_table,
                     reinterpret_cast<const uint8_t*>(a.k), reinterpret_cast<const uint8_t*>(a.v),
                     static_cast<uint16_t*>(k_dst), static_cast<uint16_t*>(v_dst), a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_merge_t(const KernelArgs& a, int n_groups, int max_rows, hipStream_t stream) {
  const int chunks = (max_rows * (D / 4) + MergeCfg<D>::THREADS - 1) / MergeCfg<D>::THREADS;
  hipLaunchKernelGGL((rpa_merge_kernel<D>), dim3(n_groups, chunks > 0 ? chunks : 1), dim3(MergeCfg<D>::THREADS), 0,
                     stream, a);
  return hipGetLastError();
}

// Prefill workgroups one compute unit holds at once: by LDS (160 KB per
// compute unit) and by waves (the waves per SIMD the shape's register budget
// is built for).
template <typename C>
constexpr int prefill_wgs_per_cu() {
  const int by_lds = (160 * 1024) / C::LDS_BYTES;
  const int by_waves = 4 * C::WAVES_PER_SIMD * 64 / C::NT;
  const int n = by_lds < by_waves ? by_lds : by_waves;
  return n > 0 ? n : 1;
}

// Prefill tile shapes per head size:
// (D, BN keys per tile, NW waves, NB 32-row blocks per wave, NS pipeline
// stages, DS waves sharing a row block by splitting d).
#define RPA_PREFILL_SHAPE_64 64, 64, 4, 2, 2, 1
#define RPA_PREFILL_SHAPE_128 128, 64, 4, 1, 2, 1
#define RPA_PREFILL_SHAPE_256 256, 32, 8, 1, 4, 1
#define RPA_PREFILL_SHAPE_512 512, 32, 8, 1, 2, 2
// Calls without decode items (the prefill launch has the compute units to
// itself), bf16 pages only.  d = 128: 32-key tiles at three waves per SIMD,
// up to 10 % faster than the shape above on windowed and chunked prefills
// (a long causal one unchanged), but beside a decode launch it leaves the
// decode workgroups fewer slots (the decode kernel 7 % slower in a mixed
// step).
#define RPA_PREFILL_SHAPE_64_ALONE RPA_PREFILL_SHAPE_64
#define RPA_PREFILL_SHAPE_128_ALONE 128, 32, 4, 1, 2, 1
#define RPA_PREFILL_SHAPE_256_ALONE RPA_PREFILL_SHAPE_256
#define RPA_PREFILL_SHAPE_512_ALONE RPA_PREFILL_SHAPE_512

// Defines the per-head-size entry points called by rpa_dispatch.cpp.
#define RPA_DEFINE_HEAD_DIM(D)                                                              \
  hipError_t launch_prefill_d##D(const KernelArgs& a, int n, bool kv8, hipStream_t s) {     \
    return launch_prefill_t<RPA_PREFILL_SHAPE_##D>(a, n, kv8, s);                          \
  }                                                                                         \
  static_assert(PrefillCfg<RPA_PREFILL_SHAPE_##D##_ALONE>::ROWS == PrefillCfg<RPA_PREFILL_SHAPE_##D>::ROWS, \
                "the prefill-only shape tiles queries like the shape of mixed steps");     \
  hipError_t launch_prefill_alone_d##D(const KernelArgs& a, int n, hipStream_t s) {         \
    return launch_prefill_t<RPA_PREFILL_SHAPE_##D##_ALONE, false>(a, n, false, s);         \
  }                                                                                         \
  hipError_t launch_decode_d##D(const KernelArgs& a, int n, int waves, bool kv8, int rows,    \
                                hipStream_t s) {                                            \
    return launch_decode_t<D>(a, n, waves, kv8, rows, s);                                   \
  }                                                                                         \
  hipError_t launch_merge_d##D(const KernelArgs& a, int n, int rows, hipStream_t s) {       \
    return launch_merge_t<D>(a, n, rows, s);                                                \
  }                                                                                         \
  hipError_t launch_append_d##D(const KernelArgs& a, int n, const void* kn, const void* vn, \
                                void* kd, void* vd, bool kv8, hipStream_t s) {              \
    return launch_append_t<D>(a, n, kn, vn, kd, vd, kv8, s);                                \
  }                                                                                         \
  hipError_t launch_stage_d##D(const KernelArgs& a, const int32_t* st, int n, void* kd,     \
                               void* vd, hipStream_t s) {                                   \
    return launch_stage_t<D>(a, st, n, kd, vd, s);                                          \
  }                                                                                         \
  int prefill_rows_d##D() { return PrefillCfg<RPA_PREFILL_SHAPE_##D>::ROWS; }              \
  int prefill_wgs_per_cu_d##D() { return prefill_wgs_per_cu<PrefillCfg<RPA_PREFILL_SHAPE_##D>>(); } \
  int prefill_fp8_tiles_d##D() { return PrefillCfg<RPA_PREFILL_SHAPE_##D, true>::CB; }     \
  int prefill_run_keys_d##D(const KernelArgs& a, bool alone) {                              \
    return alone ? prefill_run_keys<RPA_PREFILL_SHAPE_##D##_ALONE>(a, 2)                    \
                 : prefill_run_keys<RPA_PREFILL_SHAPE_##D>(a, 2);                           \
  }

}  // namespace rpa
