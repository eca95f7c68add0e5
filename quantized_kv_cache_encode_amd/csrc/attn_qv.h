// Decode attention with both keys and values stored as codes of the Hadamard/Lloyd-Max codec.
//
// Keys: "AXELRAM: Quantize Once, Never Dequantize" (Abstract): a key is stored as its norm and the b-bit
// Lloyd-Max indices of its rotated unit vector H D k / |k|; on read the query is rotated once and the
// score is |k| times the inner product of the rotated query with the codebook levels the indices select,
// with no inverse transform per key.  Values are stored with the same codec (the shift-accumulate
// attention page's English abstract also quantizes V, in a codec of its own), and the weighted sum is
// accumulated in the rotated domain: o' = sum_t p_t |v_t| c_hat_t, so the inverse transform
// o = D H o' / sum_t p_t is applied once per query head instead of once per cached value.
//
// Work decomposition (one workgroup of 8 waves per (batch b, kv head, group of GG query heads, T split),
// as in the other read kernels).  A wave takes 16-key tiles, TPC of them per chunk:
//   scores on the matrix cores: S^T[key][col] = C_hat[key][coord] . Q'^T[coord][col] with MFMA 16x16x16
//   f16; lane (r16, kq) of the A operand holds 4 code levels of key r16 from the quarter kq of its row,
//   read from a table in LDS indexed by 2 or 4 codes at a time that holds every level as an fp16 high
//   part and an fp16 low part (two products, one per part); the 16 B columns hold the GG rotated queries
//   split the same way into high parts (columns 0..7) and low parts (columns 8..15), so the two products
//   give all four partial products and a row rotation by 8 adds the halves (both operands enter with
//   about 22 significant bits);
//   the score accumulator of lane (r16, kq) holds keys 4kq..4kq+3 of head r16 & 7, which is exactly the
//   B operand layout of the AV product, so the probabilities never leave registers;
//   AV on the matrix cores: out'^T[coord][head] += V_hat^T[coord][key] . P^T[key][head]; lane (r16, kq)
//   of the A operand holds coordinate r16 * D/16 + j of keys 4kq..4kq+3: every key's levels for two
//   consecutive coordinates come from one read of a small LDS table indexed by the two codes, a byte
//   permute transposes them, and the value norms scale them (packed fp16).
// The online softmax, the wave merge and the split merge are those of the other decode kernel; the merged
// rotated-domain output goes through an in-register fast Walsh-Hadamard transform and the sign flip.
#pragma once

#include "attn_kernels.h"

namespace kvq {

template <int D_, int BITS_>
struct QvCfg {
  static constexpr int D = D_;
  static constexpr int BITS = BITS_;
  static constexpr int BPK = D * BITS / 8;      // bytes per code row
  static constexpr int FK = D * BITS / 4;       // key-code bits per lane per key (a quarter of the row)
  static constexpr int FV = D * BITS / 16;      // value-code bits per lane per key (a sixteenth)
  static constexpr int DPL = D / 16;            // value coordinates per lane (AV products per tile)
  static constexpr int KB = D / 16;             // score products per tile
  static constexpr int TPC = D <= 128 ? 4 : 2;  // 16-key tiles per chunk
  static constexpr int CH = 16 * TPC;           // keys per chunk
  static constexpr uint32_t MB = 0x01010101u * ((1u << BITS) - 1u);  // one code per byte
  // value side: every lane's field is whole bytes and codes are aligned within bytes
  static constexpr bool kFastV = BITS != 3 && FV % 8 == 0;
  // rows that are not whole 32-bit words (d = 16 with b = 1 or 3: 2 or 6 bytes) are read in 16-bit units
  static constexpr bool kHalfRows = BPK % 4 != 0;
  // key side with two codes per table entry: the entry [hi, hi, lo, lo] is the A operand itself, against a
  // B operand that repeats the two coordinates (more B registers: not for d = 256)
  static constexpr bool kKEntry = D <= 128;
  // value side from the pair table (two coordinates per lane at least)
  static constexpr bool kVPairs = DPL >= 2;
};

// A field of F bits that starts at a multiple of F bits in a code row, loaded into NF 32-bit words (the
// field's first bit at bit 0 of word 0).  Sizes of 8..256 bits are loaded exactly; other fields come from
// a window of whole words funnel-shifted by the field's bit offset within its first word.
template <int F>
struct Field {
  static constexpr bool kExact = F == 8 || F == 16 || F == 32 || F == 64 || F == 128 || F == 256;
  static constexpr int NF = (F + 31) / 32;
  static constexpr int NWIN = kExact ? NF : NF + 1;
};

// Exact fields are loaded non-temporally (each byte by one load, once per call); the windows of inexact
// fields overlap their neighbours' words and keep the default policy, which measured faster for them.
template <int F>
__device__ __forceinline__ void load_field(__amdgpu_buffer_rsrc_t r, int voff, int soff, int shift,
                                           uint32_t (&f)[Field<F>::NF]) {
  if constexpr (F == 8) {
    f[0] = __builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, kStreamLoad);
  } else if constexpr (F == 16) {
    f[0] = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kStreamLoad);
  } else if constexpr (F == 32) {
    f[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kStreamLoad);
  } else if constexpr (F == 64) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kStreamLoad);
    f[0] = x[0];
    f[1] = x[1];
  } else if constexpr (F % 128 == 0 && Field<F>::kExact) {
#pragma unroll
    for (int k = 0; k < F / 128; ++k) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff + 16 * k, kStreamLoad);
      f[4 * k + 0] = x[0];
      f[4 * k + 1] = x[1];
      f[4 * k + 2] = x[2];
      f[4 * k + 3] = x[3];
    }
  } else {
    // word-aligned window (each word its own load, so a word past the valid range reads as 0 on its own)
    uint32_t w[Field<F>::NWIN];
#pragma unroll
    for (int k = 0; k < Field<F>::NWIN; ++k) w[k] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff + 4 * k, 0);
#pragma unroll
    for (int k = 0; k < Field<F>::NF; ++k) f[k] = __builtin_amdgcn_alignbit(w[k + 1], w[k], shift);
  }
}

// A field of F <= 16 bits at a 2-byte aligned offset voff + soff, shifted right by `shift` (< 16): two
// 16-bit loads (code rows of an even number of bytes that are not whole 32-bit words).
template <int F>
__device__ __forceinline__ void load_field_h(__amdgpu_buffer_rsrc_t r, int voff, int soff, int shift, uint32_t (&f)[1]) {
  static_assert(F <= 16, "16-bit windows serve fields of up to 16 bits");
  const uint32_t h0 = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
  const uint32_t h1 = __builtin_amdgcn_raw_buffer_load_b16(r, voff + 2, soff, 0);
  f[0] = (h0 | (h1 << 16)) >> shift;
}

// Byte offset (of the word holding it, for inexact fields) and bit shift of field number idx.
template <int F>
__device__ __forceinline__ void field_pos(int idx, int& byte_off, int& shift) {
  const int bit = idx * F;
  if constexpr (Field<F>::kExact) {
    byte_off = bit / 8;
    shift = 0;
  } else {
    byte_off = (bit / 32) * 4;
    shift = bit % 32;
  }
}

// Code i (BITS bits at bit i * BITS) of a field held in NF words.
template <int BITS, int NF>
__device__ __forceinline__ uint32_t field_code(const uint32_t (&f)[NF], int i) {
  const int bit = i * BITS, w = bit / 32, o = bit % 32;
  if (o + BITS <= 32) return __builtin_amdgcn_ubfe(f[w], o, BITS);
  return __builtin_amdgcn_alignbit(f[w + 1], f[w], o) & ((1u << BITS) - 1u);
}

// N bits (N <= 16) at bit `bit` (compile-time) of a field held in NF words.
template <int N, int NF>
__device__ __forceinline__ uint32_t field_bits(const uint32_t (&f)[NF], int bit) {
  const int w = bit / 32, o = bit % 32;
  if (o + N <= 32) return __builtin_amdgcn_ubfe(f[w], o, N);
  return __builtin_amdgcn_alignbit(f[w + 1], f[w], o) & ((1u << N) - 1u);
}

// The codebook levels as fp16, split into byte planes for byte-permute lookups: lo[k] / hi[k] hold the
// low / high bytes of levels 4k .. 4k+3.
struct LevelTab {
  uint32_t lo[4], hi[4];
};

// Four codes (one per byte of sel, each < 2^BITS) -> their four fp16 levels.
template <int BITS>
__device__ __forceinline__ half4_t lookup4(uint32_t sel, const LevelTab& t) {
  uint32_t lo, hi;
  if constexpr (BITS <= 3) {
    lo = __builtin_amdgcn_perm(t.lo[1], t.lo[0], sel);
    hi = __builtin_amdgcn_perm(t.hi[1], t.hi[0], sel);
  } else {
    // levels 0..7 from the first pair of words, 8..15 from the second; bit 3 of every code picks the
    // byte of one or the other (selector byte k + 4 * bit3)
    const uint32_t s7 = sel & 0x07070707u;
    const uint32_t la = __builtin_amdgcn_perm(t.lo[1], t.lo[0], s7);
    const uint32_t lb = __builtin_amdgcn_perm(t.lo[3], t.lo[2], s7);
    const uint32_t ha = __builtin_amdgcn_perm(t.hi[1], t.hi[0], s7);
    const uint32_t hb = __builtin_amdgcn_perm(t.hi[3], t.hi[2], s7);
    const uint32_t pick = ((sel >> 1) & 0x04040404u) | 0x03020100u;
    lo = __builtin_amdgcn_perm(lb, la, pick);
    hi = __builtin_amdgcn_perm(hb, ha, pick);
  }
  typedef unsigned u2 __attribute__((ext_vector_type(2)));
  const u2 x = u2{__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u)};
  return __builtin_bit_cast(half4_t, x);
}

// Byte m of four words, as the four bytes of one word.
__device__ __forceinline__ uint32_t gather_byte(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, int m) {
  const uint32_t sel = (uint32_t)m | ((uint32_t)(4 + m) << 8) | 0x0c0c0000u;  // [a0.m, a1.m, 0, 0]
  const uint32_t x01 = __builtin_amdgcn_perm(a1, a0, sel);
  const uint32_t x23 = __builtin_amdgcn_perm(a3, a2, sel);
  return __builtin_amdgcn_perm(x23, x01, 0x05040100u);
}

// Level tables in LDS, indexed by two consecutive codes of one row (e = c0 | c1 << BITS):
//   key table, entry e = [hi(c0), hi(c1)] [lo(c0), lo(c1)] (two words: fp16 high parts, then the fp16 low
//   parts level - high part);
//   value table, entry e = [lvl(c0), lvl(c1)] (one word, fp16).
// Lookups are random, so the tables are stored 32 times over, one copy per LDS bank: word k of entry e of
// copy c sits at byte e * 256 + k * 128 + c * 4 (each entry spans 256 bytes; the value table uses the first
// half of each), and lane l reads copy l % 32, so the 32 lanes an LDS cycle serves never meet in a bank.
// With 4-bit codes the index is a whole byte of the code row, and one byte permute forms the address
// index * 256 + copy * 4 (+ the value table's base, 2^16) from the code word and the lane's copy offset.
template <int BITS>
struct LvlTabs {
  static constexpr int IB = 2 * BITS;                  // index bits
  static constexpr int NE = 1 << IB;                   // entries
  static constexpr size_t v_off = (size_t)NE * 256;    // key table first (2^16 bytes for 4-bit codes)
  static constexpr size_t bytes = 2 * v_off;
  static constexpr bool kPermAddr = BITS == 4;
};

template <class C, int GG>
struct QvPlan {
  static constexpr size_t red_bytes = (size_t)kWaves * GG * (C::D + 2) * 4;
  static constexpr size_t vtab_off = LvlTabs<C::BITS>::v_off;
  static constexpr size_t tabs_bytes = LvlTabs<C::BITS>::bytes;
  static constexpr size_t region0 = ((red_bytes > tabs_bytes ? red_bytes : tabs_bytes) + 15) / 16 * 16;
  static constexpr size_t consts_off = region0;                     // 16 levels, merge flag (+96)
  static constexpr size_t qs_off = consts_off + 128;                // GG * D floats (rotated queries)
  static constexpr size_t xs_off = qs_off + (size_t)GG * C::D * 4;  // GG * D floats (merged output)
  static constexpr size_t total = xs_off + (size_t)GG * C::D * 4;
};

template <int D, int BITS, int GG>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2))) void qv_decode_kernel(const AttnParams p) {
  using C = QvCfg<D, BITS>;
  using S = HlmScorer<D, BITS>;
  using Plan = QvPlan<C, GG>;
  constexpr int NFK = Field<C::FK>::NF, NFV = Field<C::FV>::NF;
  constexpr int DPL = C::DPL, KB = C::KB, TPC = C::TPC;
  static_assert(GG <= 8, "query heads fill half of the 16 product columns");
  __shared__ __align__(16) unsigned char smem[Plan::total];
  float* lv = reinterpret_cast<float*>(smem + Plan::consts_off);
  int* s_flag = reinterpret_cast<int*>(smem + Plan::consts_off + 96);
  float* qs = reinterpret_cast<float*>(smem + Plan::qs_off);
  float* xs = reinterpret_cast<float*>(smem + Plan::xs_off);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, kq = lane >> 4;
  const Unit u = decode_unit(p, GG);
  const int split = blockIdx.x;
  const int64_t t_begin = (int64_t)split * p.split_len;
  int64_t t_end = t_begin + p.split_len;
  if (t_end > u.len) t_end = u.len;
  const int n_valid = t_end > t_begin ? (int)(t_end - t_begin) : 0;
  const int64_t rowb = ((int64_t)u.b * p.Hkv + u.kvh) * p.T_cap + t_begin;
  const __amdgpu_buffer_rsrc_t rkc = make_rsrc(p.codes + (size_t)rowb * C::BPK, (int64_t)n_valid * C::BPK);
  const __amdgpu_buffer_rsrc_t rkn = make_rsrc(p.norms + rowb, (int64_t)n_valid * 4);
  const __amdgpu_buffer_rsrc_t rvc = make_rsrc(p.vcodes + (size_t)rowb * C::BPK, (int64_t)n_valid * C::BPK);
  const __amdgpu_buffer_rsrc_t rvn = make_rsrc(p.vnorms + rowb, (int64_t)n_valid * 4);
  // per-lane offsets (fixed for the loop): key side = key r16 of a tile, quarter kq of its row; value side
  // = keys 4kq..4kq+3 of a tile, sixteenth r16 of their rows; norms of keys 4kq..4kq+3
  int kbyte, kshift, vbyte, vshift;
  field_pos<C::FK>(kq, kbyte, kshift);
  field_pos<C::FV>(r16, vbyte, vshift);
  int voff_k = r16 * C::BPK + kbyte;
  const int voff_v = 4 * kq * C::BPK + vbyte;
  const int voff_n = 4 * kq * 4;
  // 16-bit windows: byte offset and shift from the field's bit position within the whole split
  int hoff_v[4] = {0, 0, 0, 0}, hsh_v[4] = {0, 0, 0, 0};
  if constexpr (C::kHalfRows) {
    const int kb = r16 * C::BPK * 8 + kq * C::FK;
    voff_k = (kb / 16) * 2;
    kshift = kb % 16;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int vb = (4 * kq + s) * C::BPK * 8 + r16 * C::FV;
      hoff_v[s] = (vb / 16) * 2;
      hsh_v[s] = vb % 16;
    }
  }

  struct Chunk {
    uint32_t kc[TPC][NFK];
    uint32_t vc[TPC][4][NFV];
    float4_t kn[TPC], vn[TPC];
  };
  auto fetch = [&](int cc, Chunk& k) {
#pragma unroll
    for (int t = 0; t < TPC; ++t) {
      const int row = cc + 16 * t;
      if constexpr (C::kHalfRows) {
        load_field_h<C::FK>(rkc, voff_k, row * C::BPK, kshift, k.kc[t]);
#pragma unroll
        for (int s = 0; s < 4; ++s) load_field_h<C::FV>(rvc, hoff_v[s], row * C::BPK, hsh_v[s], k.vc[t][s]);
      } else {
        load_field<C::FK>(rkc, voff_k, row * C::BPK, kshift, k.kc[t]);
#pragma unroll
        for (int s = 0; s < 4; ++s) load_field<C::FV>(rvc, voff_v, (row + s) * C::BPK, vshift, k.vc[t][s]);
      }
      k.kn[t] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(rkn, voff_n, row * 4, kStreamLoad));
      k.vn[t] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(rvn, voff_n, row * 4, kStreamLoad));
    }
  };
  constexpr int STR = kWaves * C::CH;
  int c = wid * C::CH;
  Chunk ka, kb;
  prologue<S, GG>(p, u, qs, nullptr, lv, tid, [&] { fetch(c, ka); });

  // fp16 level tables (from LDS, so they live in vector registers as the permutes need)
  LevelTab tab;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)lv[4 * k + e]);
      lo |= (h & 0xffu) << (8 * e);
      hi |= (h >> 8) << (8 * e);
    }
    tab.lo[k] = lo;
    tab.hi[k] = hi;
  }
  // level tables (the table region is free until the wave merge): every thread makes one word of one
  // entry and writes its 32 copies (128 contiguous bytes)
  using LT = LvlTabs<BITS>;
  unsigned char* vtab = smem + Plan::vtab_off;
  {
    typedef unsigned u4w __attribute__((ext_vector_type(4)));
    // the 8 stores of a lane start at different 16-byte quarters of its run, so that the lanes of one store
    // spread over all banks (runs are 128 bytes apart, i.e. in the same banks)
    auto put32 = [&](unsigned char* dst, uint32_t w) {
#pragma unroll
      for (int k = 0; k < 8; ++k) *reinterpret_cast<u4w*>(dst + 16 * ((k + lane) & 7)) = u4w{w, w, w, w};
    };
    auto pack2 = [](_Float16 a, _Float16 b) -> uint32_t {
      return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
    };
    for (int x = tid; x < LT::NE * 2; x += kThreads) {  // key table: x = entry * 2 + part
      const int e = x >> 1, part = x & 1;                  // part 0: high parts, 1: low parts
      const float l0 = lv[e & ((1 << BITS) - 1)], l1 = lv[e >> BITS];
      const _Float16 h0 = (_Float16)l0, h1 = (_Float16)l1;
      const uint32_t w = part ? pack2((_Float16)(l0 - (float)h0), (_Float16)(l1 - (float)h1)) : pack2(h0, h1);
      put32(smem + (size_t)x * 128, w);
    }
    if constexpr (C::kVPairs) {
      for (int e = tid; e < LT::NE; e += kThreads)
        put32(vtab + (size_t)e * 256, pack2((_Float16)lv[e & ((1 << BITS) - 1)], (_Float16)lv[e >> BITS]));
    }
  }
  const uint32_t bank4 = (uint32_t)(lane & 31) * 4;  // this lane's copy
  const uint32_t bank4v = bank4 | (uint32_t)Plan::vtab_off;
  // byte address of entry idx: idx * 256 + base, idx the IB bits at bit `bit` of a field
  auto ent_addr = [&](const auto& f, int bit, uint32_t base) -> uint32_t {
    if constexpr (LT::kPermAddr) {
      // [base.b0, code byte, base.b2, 0] (base < 2^24 with a zero second byte)
      const int w = bit / 32, m = (bit % 32) / 8;
      return __builtin_amdgcn_perm(f[w], base, 0x0c020400u | ((uint32_t)(4 + m) << 8));
    } else {
      return base + field_bits<LT::IB, sizeof(f) / 4>(f, bit) * 256u;
    }
  };
  // B operands of the score products: column r16 holds head r16 & 7, high part (r16 < 8) or low part.
  // Slot m of product kb holds the coordinate of code slot_code(kb, m) of this lane's quarter row.
  constexpr int NBQ = C::kKEntry ? D / 8 : KB;
  half4_t bq[NBQ];
  {
    const int g = r16 & 7;
#pragma unroll
    for (int kb = 0; kb < NBQ; ++kb) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int code = C::kKEntry ? 2 * kb + (m & 1) : 4 * kb + m;
        _Float16 v = 0;
        if (g < GG) {
          const float x = qs[g * D + kq * (D / 4) + code];
          const _Float16 h = (_Float16)x;
          v = r16 < 8 ? h : (_Float16)(x - (float)h);
        }
        bq[kb][m] = v;
      }
    }
  }

  lds_barrier();  // the key-level table is complete

  float m_run = -INFINITY, l_lane = 0.0f;
  float4_t oacc[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) oacc[j] = float4_t{0.f, 0.f, 0.f, 0.f};

  auto process = [&](int cc, Chunk& k) {
    // ---- scores of the chunk's tiles (keys 4kq+i of tile t, head r16 & 7)
    float z[TPC][4];
#pragma unroll
    for (int t = 0; t < TPC; ++t) {
      // A operands: levels of this lane's quarter row from the key table, high and low parts
      float4_t acc = float4_t{0.f, 0.f, 0.f, 0.f};
      typedef unsigned u2 __attribute__((ext_vector_type(2)));
      auto kent = [&](uint32_t addr) -> u2 {
        const unsigned char* a = smem + addr;
        return u2{*reinterpret_cast<const uint32_t*>(a), *reinterpret_cast<const uint32_t*>(a + 128)};
      };
      if constexpr (C::kKEntry) {
        // one entry = [hi(c), hi(c')] [lo(c), lo(c')] of codes 2e, 2e+1: a whole operand
#pragma unroll
        for (int e2 = 0; e2 < D / 8; ++e2) {
          const u2 ent = kent(ent_addr(k.kc[t], 2 * e2 * BITS, bank4));
          acc = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, ent), bq[e2], acc, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int kb2 = 0; kb2 < KB; ++kb2) {
          const u2 e0 = kent(ent_addr(k.kc[t], 4 * kb2 * BITS, bank4));
          const u2 e1 = kent(ent_addr(k.kc[t], (4 * kb2 + 2) * BITS, bank4));
          const half4_t ahi = __builtin_bit_cast(half4_t, u2{e0[0], e1[0]});
          const half4_t alo = __builtin_bit_cast(half4_t, u2{e0[1], e1[1]});
          acc = __builtin_amdgcn_mfma_f32_16x16x16f16(ahi, bq[kb2], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x16f16(alo, bq[kb2], acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = acc[i] + dpp_f<0x128>(acc[i]);  // row_ror:8 -- high part + low part
        z[t][i] = s * (k.kn[t][i] * p.zscale);
      }
    }
    if (cc + C::CH > n_valid) {  // the split's last, partial chunk
#pragma unroll
      for (int t = 0; t < TPC; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) z[t][i] = cc + 16 * t + 4 * kq + i < n_valid ? z[t][i] : -INFINITY;
    }
    // ---- online softmax with the lazily raised maximum (probabilities stay <= 2^8)
    float zmax = z[0][0];
#pragma unroll
    for (int t = 0; t < TPC; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) zmax = fmaxf(zmax, z[t][i]);
    if (__any(zmax - m_run > kLazyHeadroom)) {
      float mx = fmaxf(zmax, __shfl_xor(zmax, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - mn);
      m_run = mn;
      l_lane *= alpha;
#pragma unroll
      for (int j = 0; j < DPL; ++j) oacc[j] *= alpha;
    }
#pragma unroll
    for (int t = 0; t < TPC; ++t) {
      half4_t pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pr = fast_exp2(z[t][i] - m_run);
        l_lane += pr;
        pb[i] = (_Float16)pr;
      }
      // ---- value levels: coordinate r16 * DPL + j of keys 4kq..4kq+3, times the value norms
      typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
      const half2_t n01 = half2_t{(_Float16)k.vn[t][0], (_Float16)k.vn[t][1]};
      const half2_t n23 = half2_t{(_Float16)k.vn[t][2], (_Float16)k.vn[t][3]};
      if constexpr (C::kVPairs) {
        // coordinates 2pm and 2pm+1 of each of the four keys from the pair table, then a 2 x 4 transpose
#pragma unroll
        for (int pm = 0; pm < DPL / 2; ++pm) {
          uint32_t e[4];
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
            e[s2] = *reinterpret_cast<const uint32_t*>(smem + ent_addr(k.vc[t][s2], 2 * pm * BITS, bank4v));
          typedef unsigned u2 __attribute__((ext_vector_type(2)));
          const half4_t lo4 = __builtin_bit_cast(half4_t, u2{__builtin_amdgcn_perm(e[1], e[0], 0x05040100u),
                                                             __builtin_amdgcn_perm(e[3], e[2], 0x05040100u)});
          const half4_t hi4 = __builtin_bit_cast(half4_t, u2{__builtin_amdgcn_perm(e[1], e[0], 0x07060302u),
                                                             __builtin_amdgcn_perm(e[3], e[2], 0x07060302u)});
          const half2_t a01 = half2_t{lo4[0], lo4[1]} * n01, a23 = half2_t{lo4[2], lo4[3]} * n23;
          const half2_t b01 = half2_t{hi4[0], hi4[1]} * n01, b23 = half2_t{hi4[2], hi4[3]} * n23;
          oacc[2 * pm] = __builtin_amdgcn_mfma_f32_16x16x16f16(half4_t{a01[0], a01[1], a23[0], a23[1]}, pb,
                                                               oacc[2 * pm], 0, 0, 0);
          oacc[2 * pm + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(half4_t{b01[0], b01[1], b23[0], b23[1]}, pb,
                                                                   oacc[2 * pm + 1], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
          uint32_t sel;
          if constexpr (C::kFastV) {
            const int bit = j * BITS, m = bit / 8, wi = m / 4;
            const uint32_t g = gather_byte(k.vc[t][0][wi], k.vc[t][1][wi], k.vc[t][2][wi], k.vc[t][3][wi], m % 4);
            sel = (g >> (bit % 8)) & C::MB;
          } else {
            sel = field_code<BITS, NFV>(k.vc[t][0], j) | (field_code<BITS, NFV>(k.vc[t][1], j) << 8) |
                  (field_code<BITS, NFV>(k.vc[t][2], j) << 16) | (field_code<BITS, NFV>(k.vc[t][3], j) << 24);
          }
          const half4_t lvl = lookup4<BITS>(sel, tab);
          const half2_t v01 = half2_t{lvl[0], lvl[1]} * n01;
          const half2_t v23 = half2_t{lvl[2], lvl[3]} * n23;
          const half4_t av = half4_t{v01[0], v01[1], v23[0], v23[1]};
          oacc[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, pb, oacc[j], 0, 0, 0);
        }
      }
    }
  };

  for (; c < n_valid; c += 2 * STR) {
    fetch(c + STR, kb);
    process(c, ka);
    if (c + STR >= n_valid) break;
    fetch(c + 2 * STR, ka);
    process(c + STR, kb);
  }

  // ---- merge the waves through LDS: rotated-domain accumulators, maxima and sums per head
  float l_w = l_lane + __shfl_xor(l_lane, 16, 64);
  l_w += __shfl_xor(l_w, 32, 64);  // the head's sum over this wave (lanes r16 and r16 + 8 hold the same)
  lds_barrier();
  float* red = reinterpret_cast<float*>(smem);  // [kWaves][GG][D]
  float* red_m = red + kWaves * GG * D;          // [kWaves][GG]
  float* red_l = red_m + kWaves * GG;            // [kWaves][GG]
  if (r16 < GG) {
#pragma unroll
    for (int j = 0; j < DPL; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(wid * GG + r16) * D + DPL * (4 * kq + r) + j] = oacc[j][r];
    if (kq == 0) {
      red_m[wid * GG + r16] = m_run;
      red_l[wid * GG + r16] = l_w;
    }
  }
  lds_barrier();
  const bool split_merge = p.n_splits > 1;
  float* mine_m = qs;       // [GG] this workgroup's merged maxima and totals (the rotated queries are no
  float* mine_d = qs + GG;  // longer needed); its merged sums go to xs
  if (split_merge && tid == 0) *s_flag = merger_from_count(p.counters + blockIdx.y, count_arrival(p.counters + blockIdx.y), p.n_splits);
  for (int idx = tid; idx < GG * D; idx += kThreads) {
    const int g = idx / D, dc = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) M = fmaxf(M, red_m[w2 * GG + g]);
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2) {
        const float wt = fast_exp2(red_m[w2 * GG + g] - M);
        num += wt * red[(w2 * GG + g) * D + dc];
        den += wt * red_l[w2 * GG + g];
      }
    }
    if (!split_merge) {
      xs[idx] = den > 0.0f ? num / den : 0.0f;
    } else {
      xs[idx] = num;
      if (dc == 0) {
        mine_m[g] = M;
        mine_d[g] = den;
      }
    }
  }
  if (split_merge) {
    // ---- every workgroup but the last publishes its partials; the last merges all splits
    lds_barrier();
    const bool last = *s_flag;
    uint32_t* wsw = reinterpret_cast<uint32_t*>(p.ws);
    for (int idx = tid; idx < GG * D; idx += kThreads) {
      const int g = idx / D, dc = idx % D;
      const size_t row = (size_t)u.b * p.Hq + u.h0 + g;
      uint32_t* base = wsw + row * (size_t)p.n_splits * (D + kRecPad);
      float M = mine_m[g], num = xs[idx], den = mine_d[g];
      if (!last) {
        publish_partial<D>(base + (size_t)split * (D + kRecPad), dc, num, M, den);
        continue;
      }
      merge_partials<D>(base, p.n_splits, split, dc, M, num, den);
      xs[idx] = den > 0.0f ? num / den : 0.0f;
    }
    if (!last) return;
    __syncthreads();  // every thread of the merger has read its words
    for (int idx = tid; idx < GG * D; idx += kThreads) {
      const int g = idx / D, dc = idx % D;
      const size_t row = (size_t)u.b * p.Hq + u.h0 + g;
      clear_partials<D>(wsw + row * (size_t)p.n_splits * (D + kRecPad), p.n_splits, split, dc);
    }
  }
  lds_barrier();

  // ---- back to the original domain once per head: o = D H o' (H normalised, Sylvester order)
  constexpr int LPQ = D / 8;  // lanes per head, 8 coordinates each
  static_assert(GG * LPQ <= kThreads, "one lane per 8 coordinates of every head");
  const int g = tid / LPQ, kk = tid % LPQ;
  if (g < GG) {  // whole groups of LPQ lanes (LPQ divides 64), so the cross-lane steps stay in the group
    float x[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) x[t] = xs[g * D + 8 * kk + t];
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if ((t & h) == 0) {
          const float a = x[t], b = x[t + h];
          x[t] = a + b;
          x[t + h] = a - b;
        }
#pragma unroll
    for (int dl = 1; dl < LPQ; dl <<= 1) {
      const bool upper = (kk & dl) != 0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float o = __shfl_xor(x[t], dl, 64);
        x[t] = upper ? (o - x[t]) : (x[t] + o);
      }
    }
    const float rs = 1.0f / __builtin_sqrtf((float)D);
    uint32_t sw = 0;  // the sign word of these coordinates, picked with uniform reads of the arguments
#pragma unroll
    for (int w = 0; w < (D + 31) / 32; ++w)
      if (((8 * kk) >> 5) == w) sw = p.signs[w];
    const uint32_t sb = (sw >> ((8 * kk) & 31)) & 0xffu;
    const size_t row = (size_t)u.b * p.Hq + u.h0 + g;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float o = ((sb >> t) & 1u) ? -x[t] * rs : x[t] * rs;
      if (p.out_f16) reinterpret_cast<_Float16*>(p.out)[row * D + 8 * kk + t] = (_Float16)o;
      else reinterpret_cast<float*>(p.out)[row * D + 8 * kk + t] = o;
    }
  }
}

template <int D, int BITS>
hipError_t run_qv_decode_bits(int gg, const AttnParams& p, dim3 grid, hipStream_t s) {
  using C = QvCfg<D, BITS>;
  switch (gg) {
    case 1: return launch_attn(qv_decode_kernel<D, BITS, 1>, QvPlan<C, 1>::total, grid, s, p);
    case 2: return launch_attn(qv_decode_kernel<D, BITS, 2>, QvPlan<C, 2>::total, grid, s, p);
    case 4: return launch_attn(qv_decode_kernel<D, BITS, 4>, QvPlan<C, 4>::total, grid, s, p);
    case 8: return launch_attn(qv_decode_kernel<D, BITS, 8>, QvPlan<C, 8>::total, grid, s, p);
    default: return hipErrorNotSupported;
  }
}

template <int D>
hipError_t run_qv_decode(int bits, int gg, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (bits) {
    case 1: return run_qv_decode_bits<D, 1>(gg, p, grid, s);
    case 2: return run_qv_decode_bits<D, 2>(gg, p, grid, s);
    case 3: return run_qv_decode_bits<D, 3>(gg, p, grid, s);
    case 4: return run_qv_decode_bits<D, 4>(gg, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace kvq
