// Radix keys for multimodal inputs.
//
// For RadixAttention on multimodal models, the runtime hashes each input
// image and uses the hash as the key in the radix tree, so the KV of the
// image tokens of the same image is reused (unite.ai, "SGLang: Efficient
// Execution of Structured Language Model Programs", section "Resultados en
// modelos multimodales").  The tree here is keyed by int32 token ids, so an
// image that occupies n positions of a request becomes n keys:
//   hash   = 64-bit FNV-1a of the image bytes (offset basis
//            0xcbf29ce484222325, prime 0x100000001b3);
//   key[i] = -1 - (splitmix64(hash + (i + 1) * 0x9e3779b97f4a7c15) >> 33),
// i.e. the splitmix64 finalizer on a Weyl sequence seeded by the hash.  Keys
// lie in [-2^31, -1], disjoint from text ids (>= 0); they depend on the
// position, so a match that ends inside an image stops at the same position
// for every request holding it, and two different images already differ at
// their first key unless 31 hash-derived bits collide.

#include <stdint.h>

#include "rkv.h"
#include "rkv_internal.h"

namespace {

uint64_t fnv1a64(const uint8_t* p, int64_t n) {
  uint64_t h = 0xcbf29ce484222325ull;
  for (int64_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 0x100000001b3ull;
  }
  return h;
}

uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

}  // namespace

extern "C" int rkv_image_keys(const uint8_t* bytes, int64_t len, int64_t n_tokens, int32_t* keys,
                              uint64_t* out_hash) {
  rkv::clear_error();
  if (len < 0 || n_tokens < 0 || (len > 0 && !bytes) || (n_tokens > 0 && !keys))
    return rkv::fail(RKV_EINVAL, "rkv_image_keys: bad argument");
  const uint64_t h = fnv1a64(bytes, len);
  for (int64_t i = 0; i < n_tokens; ++i) {
    const uint64_t z = mix64(h + (uint64_t)(i + 1) * 0x9e3779b97f4a7c15ull);
    keys[i] = (int32_t)(-1 - (int64_t)(z >> 33));
  }
  if (out_hash) *out_hash = h;
  return RKV_OK;
}
