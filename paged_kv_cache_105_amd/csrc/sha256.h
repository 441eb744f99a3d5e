// SHA-256 (FIPS 180-4), used for chained block identities of the prefix
// cache.  Streaming interface: init, update any number of times, final.
#pragma once

#include <cstddef>
#include <cstdint>

namespace pkv {

struct Sha256 {
  uint32_t h[8];
  uint8_t buf[64];
  uint64_t len = 0;  // bytes absorbed
  size_t fill = 0;   // bytes in buf

  Sha256();
  void update(const void* data, size_t n);
  void final(uint8_t out[32]);

 private:
  void block(const uint8_t* p);
};

}  // namespace pkv
