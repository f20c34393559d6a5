// prepack.cpp -- host-side repack of standard-format weights into the kernels' MFMA operand
// layout (layout.h). Pure C++, no HIP calls: it runs once per weight at load time, as the
// preprocessing step of the Humming announcement (section "Tuning and JIT compilation per
// workload": validate, pad, repack into the target kernel's layout).
#include <algorithm>
#include <cstring>
#include <thread>
#include <vector>

#include "internal.h"
#include "layout.h"

namespace hq {
namespace {

// Parallel loop over [0, n) in contiguous chunks; the work is memory-bound byte shuffling.
template <class F>
void parallel_for(int64_t n, F&& f) {
  unsigned hw = std::max(1u, std::thread::hardware_concurrency());
  int64_t workers = std::min<int64_t>(std::min<int64_t>(hw, 32), n);
  if (workers <= 1) {
    for (int64_t i = 0; i < n; ++i) f(i);
    return;
  }
  std::vector<std::thread> th;
  th.reserve(workers);
  for (int64_t w = 0; w < workers; ++w) {
    th.emplace_back([&, w] {
      for (int64_t i = w; i < n; i += workers) f(i);
    });
  }
  for (auto& t : th) t.join();
}

// Nibble j (0..7) of an 8-code group moves to slot p with j = 2*(p&3) + (p>>2).
inline uint32_t interleave8(const uint8_t* c /* 8 codes, values 0..15 */) {
  uint32_t v = 0;
  for (int p = 0; p < 8; ++p) {
    int j = 2 * (p & 3) + (p >> 2);
    v |= uint32_t(c[j] & 0xF) << (4 * p);
  }
  return v;
}

void pack_wna16(const PackedLayout& L, bool sym, const uint8_t* wq, const uint16_t* scales,
                const uint8_t* zeros, uint8_t* out) {
  const int64_t K = L.K, G = K / 128;
  parallel_for(L.n_tiles, [&](int64_t nt) {
    uint8_t codes[32];
    for (int64_t kt = 0; kt < L.k_units; ++kt) {
      uint8_t* unit = out + L.codes_off + (size_t(nt) * L.k_units + kt) * kUnitBytes;
      for (int l = 0; l < 64; ++l) {
        int64_t n = nt * 16 + (l & 15);
        int64_t k0 = kt * 128 + 32 * (l >> 4);
        const uint8_t* row = wq + size_t(n) * (K / 2);
        for (int j = 0; j < 32; ++j) {
          int64_t k = k0 + j;
          uint8_t b = row[k >> 1];
          uint8_t c = (k & 1) ? (b >> 4) : (b & 0xF);
          codes[j] = sym ? uint8_t(c ^ 0x8) : c;
        }
        uint32_t* dst = reinterpret_cast<uint32_t*>(unit + 16 * l);
        for (int d = 0; d < 4; ++d) dst[d] = interleave8(codes + 8 * d);
      }
      uint16_t* sdst = reinterpret_cast<uint16_t*>(out + L.scales_off) + (size_t(nt) * L.k_units + kt) * 16;
      for (int i = 0; i < 16; ++i) sdst[i] = scales[size_t(nt * 16 + i) * G + kt];
      if (!sym) {
        uint8_t* zdst = out + L.zeros_off + (size_t(nt) * L.k_units + kt) * 8;
        for (int i = 0; i < 8; ++i) {
          uint8_t lo = zeros[size_t(nt * 16 + 2 * i) * G + kt] & 0xF;
          uint8_t hi = zeros[size_t(nt * 16 + 2 * i + 1) * G + kt] & 0xF;
          zdst[i] = uint8_t(lo | (hi << 4));
        }
      }
    }
  });
}

// 2-bit codes (layout.h, WNA2): input wq [N, K/4] (code k in bits 2 (k % 4) of byte k / 4);
// scales and zeros as WNA16's.
void pack_wna2(const PackedLayout& L, const uint8_t* wq, const uint16_t* scales, const uint8_t* zeros,
               uint8_t* out) {
  const int64_t K = L.K, G = K / 128;
  parallel_for(L.n_tiles, [&](int64_t nt) {
    for (int64_t kt = 0; kt < L.k_units; ++kt) {
      uint8_t* unit = out + L.codes_off + (size_t(nt) * L.k_units + kt) * 512;
      for (int l = 0; l < 64; ++l) {
        const int64_t n = nt * 16 + (l & 15);
        const uint8_t* row = wq + size_t(n) * (K / 4);
        uint32_t* dst = reinterpret_cast<uint32_t*>(unit + 8 * l);
        for (int h = 0; h < 2; ++h) {
          uint32_t v = 0;
          for (int c = 0; c < 16; ++c) {
            const int64_t k = kt * 128 + 32 * (l >> 4) + 16 * h + c;
            const uint32_t code = (row[k >> 2] >> (2 * (k & 3))) & 3u;
            v |= code << (16 * (c & 1) + 2 * (c >> 1));
          }
          dst[h] = v;
        }
      }
      uint16_t* sdst = reinterpret_cast<uint16_t*>(out + L.scales_off) + (size_t(nt) * L.k_units + kt) * 16;
      for (int i = 0; i < 16; ++i) sdst[i] = scales[size_t(nt * 16 + i) * G + kt];
      uint8_t* zdst = out + L.zeros_off + (size_t(nt) * L.k_units + kt) * 8;
      for (int i = 0; i < 8; ++i) {
        const uint8_t lo = zeros[size_t(nt * 16 + 2 * i) * G + kt] & 0x3;
        const uint8_t hi = zeros[size_t(nt * 16 + 2 * i + 1) * G + kt] & 0x3;
        zdst[i] = uint8_t(lo | (hi << 4));
      }
    }
  });
}

// 3-bit codes (layout.h, WNA3): input wq [N, 3K/8], each row a little-endian bit string with
// code k in bits 3k .. 3k + 2; scales and zeros as WNA16's.
void pack_wna3(const PackedLayout& L, const uint8_t* wq, const uint16_t* scales, const uint8_t* zeros,
               uint8_t* out) {
  const int64_t K = L.K, G = K / 128;
  parallel_for(L.n_tiles, [&](int64_t nt) {
    for (int64_t kt = 0; kt < L.k_units; ++kt) {
      uint8_t* unit = out + L.codes_off + (size_t(nt) * L.k_units + kt) * 768;
      for (int l = 0; l < 64; ++l) {
        const int64_t n = nt * 16 + (l & 15);
        const uint8_t* row = wq + size_t(n) * (K / 8 * 3);
        uint32_t lo[2] = {0, 0}, hi = 0;
        for (int h = 0; h < 2; ++h)
          for (int c = 0; c < 16; ++c) {
            const int64_t k = kt * 128 + 32 * (l >> 4) + 16 * h + c;
            uint32_t code = 0;
            for (int b = 0; b < 3; ++b) {
              const int64_t bit = 3 * k + b;
              code |= uint32_t((row[bit >> 3] >> (bit & 7)) & 1u) << b;
            }
            const int s = c >> 1, e = c & 1;
            lo[h] |= (code & 3u) << (16 * e + 2 * s);
            hi |= (code >> 2) << (16 * e + 8 * h + s);
          }
        std::memcpy(unit + 8 * l, lo, 8);
        std::memcpy(unit + 512 + 4 * l, &hi, 4);
      }
      uint16_t* sdst = reinterpret_cast<uint16_t*>(out + L.scales_off) + (size_t(nt) * L.k_units + kt) * 16;
      for (int i = 0; i < 16; ++i) sdst[i] = scales[size_t(nt * 16 + i) * G + kt];
      uint8_t* zdst = out + L.zeros_off + (size_t(nt) * L.k_units + kt) * 8;
      for (int i = 0; i < 8; ++i) {
        const uint8_t zlo = zeros[size_t(nt * 16 + 2 * i) * G + kt] & 0x7;
        const uint8_t zhi = zeros[size_t(nt * 16 + 2 * i + 1) * G + kt] & 0x7;
        zdst[i] = uint8_t(zlo | (zhi << 4));
      }
    }
  });
}

void pack_w8a8(const PackedLayout& L, const int8_t* wq, const float* scales, uint8_t* out) {
  const int64_t K = L.K;
  parallel_for(L.n_tiles, [&](int64_t nt) {
    for (int64_t kt = 0; kt < L.k_units; ++kt) {
      uint8_t* unit = out + L.codes_off + (size_t(nt) * L.k_units + kt) * kUnitBytes;
      for (int l = 0; l < 64; ++l) {
        int64_t n = nt * 16 + (l & 15);
        int64_t k0 = kt * 64 + 16 * (l >> 4);
        std::memcpy(unit + 16 * l, wq + size_t(n) * K + k0, 16);
      }
    }
  });
  if (scales) std::memcpy(out + L.scales_off, scales, size_t(L.N) * 4);
}

void pack_fp8b(const PackedLayout& L, const uint8_t* wq, const float* scales, uint8_t* out) {
  const int64_t K = L.K, G = K / 128;
  pack_w8a8(L, reinterpret_cast<const int8_t*>(wq), nullptr, out);   // the codes: W8A8's units
  parallel_for(L.n_tiles, [&](int64_t nt) {
    for (int64_t g = 0; g < G; ++g) {
      const float s = scales[size_t(nt * 16 / 128) * G + g];
      float* dst = reinterpret_cast<float*>(out + L.scales_off + (size_t(nt) * G + g) * 16);
      for (int i = 0; i < 4; ++i) dst[i] = s;
    }
  });
}

// 8-bit codes for the bf16 MFMA (layout.h, W8A16 / F8A16): unit j of step kt, lane l, byte b
// holds k = 128 kt + 32 (l >> 4) + 16 j + b of channel 16 nt + (l & 15).
void pack_w8a16(const PackedLayout& L, const uint8_t* wq, const float* scales, uint8_t* out) {
  const int64_t K = L.K;
  parallel_for(L.n_tiles, [&](int64_t nt) {
    for (int64_t u = 0; u < L.k_units; ++u) {
      const int64_t kt = u >> 1, j = u & 1;
      uint8_t* unit = out + L.codes_off + (size_t(nt) * L.k_units + u) * kUnitBytes;
      for (int l = 0; l < 64; ++l) {
        const int64_t n = nt * 16 + (l & 15);
        const int64_t k0 = kt * 128 + 32 * (l >> 4) + 16 * j;
        std::memcpy(unit + 16 * l, wq + size_t(n) * K + k0, 16);
      }
    }
  });
  std::memcpy(out + L.scales_off, scales, size_t(L.N) * 4);
}

void pack_w4a8(const PackedLayout& L, const uint8_t* wq, const uint8_t* scales, uint8_t* out) {
  const int64_t K = L.K, B = K / 32;
  parallel_for(L.n_tiles, [&](int64_t nt) {
    for (int64_t kt = 0; kt < L.k_units; ++kt) {
      uint8_t* unit = out + L.codes_off + (size_t(nt) * L.k_units + kt) * kUnitBytes;
      uint8_t* sdst = out + L.scales_off + (size_t(nt) * L.k_units + kt) * 64;
      for (int l = 0; l < 64; ++l) {
        int64_t n = nt * 16 + (l & 15);
        int64_t blk = kt * 4 + (l >> 4);
        std::memcpy(unit + 16 * l, wq + size_t(n) * (K / 2) + blk * 16, 16);
        sdst[l] = scales[size_t(n) * B + blk];
      }
    }
  });
}

}  // namespace

size_t prepacked_bytes(const Combo& c, int64_t E, int64_t N, int64_t K) {
  PackedLayout L = make_layout(c.fam, c.asym, N, K);
  return L.expert_stride * size_t(E);
}

void prepack(const Combo& c, int64_t E, int64_t N, int64_t K, const void* wq,
             const void* scales, const void* zeros, void* out) {
  PackedLayout L = make_layout(c.fam, c.asym, N, K);
  std::memset(out, 0, L.expert_stride * size_t(E));
  for (int64_t e = 0; e < E; ++e) {
    uint8_t* o = static_cast<uint8_t*>(out) + L.expert_stride * size_t(e);
    if (c.fam == FAM_WNA16) {
      const size_t wq_stride = size_t(N) * (K / 2), s_stride = size_t(N) * (K / 128);
      pack_wna16(L, !c.asym, static_cast<const uint8_t*>(wq) + e * wq_stride,
                 static_cast<const uint16_t*>(scales) + e * s_stride,
                 c.asym ? static_cast<const uint8_t*>(zeros) + e * s_stride : nullptr, o);
    } else if (c.fam == FAM_WNA2) {
      const size_t s_stride = size_t(N) * (K / 128);
      pack_wna2(L, static_cast<const uint8_t*>(wq) + e * size_t(N) * (K / 4),
                static_cast<const uint16_t*>(scales) + e * s_stride, static_cast<const uint8_t*>(zeros) + e * s_stride, o);
    } else if (c.fam == FAM_WNA3) {
      const size_t s_stride = size_t(N) * (K / 128);
      pack_wna3(L, static_cast<const uint8_t*>(wq) + e * size_t(N) * (K / 8 * 3),
                static_cast<const uint16_t*>(scales) + e * s_stride, static_cast<const uint8_t*>(zeros) + e * s_stride, o);
    } else if (c.fam == FAM_W8A8) {
      pack_w8a8(L, static_cast<const int8_t*>(wq) + e * size_t(N) * K,
                static_cast<const float*>(scales) + e * size_t(N), o);
    } else if (c.fam == FAM_W8A16 || c.fam == FAM_F8A16) {
      pack_w8a16(L, static_cast<const uint8_t*>(wq) + e * size_t(N) * K,
                 static_cast<const float*>(scales) + e * size_t(N), o);
    } else if (c.fam == FAM_FP8B) {
      pack_fp8b(L, static_cast<const uint8_t*>(wq) + e * size_t(N) * K,
                static_cast<const float*>(scales) + e * size_t(N / 128) * (K / 128), o);
    } else {
      pack_w4a8(L, static_cast<const uint8_t*>(wq) + e * size_t(N) * (K / 2),
                static_cast<const uint8_t*>(scales) + e * size_t(N) * (K / 32), o);
    }
  }
}

}  // namespace hq
