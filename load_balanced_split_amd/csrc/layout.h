// Word offsets inside a task map (the layout is documented in hpcattn.h).
// Plain constexpr C++ with no HIP dependency: the host validation unit and
// the kernels share it (constexpr functions are callable from device code).
#pragma once

#include <stdint.h>

namespace hpcattn {

struct MapLayout {
    int64_t lens, bin_off, seg_off, desc, words;
    constexpr MapLayout(int32_t B, int32_t Hkv, int32_t P)
        : lens(8),
          bin_off(8 + (int64_t)B),
          seg_off(8 + (int64_t)B + (int64_t)P + 1),
          desc(8 + (int64_t)B + (int64_t)P + 1 + (int64_t)B * Hkv + 1),
          words(8 + (int64_t)B + (int64_t)P + 1 + (int64_t)B * Hkv + 1 +
                4 * ((int64_t)B * Hkv + P - 1)) {}
};

}  // namespace hpcattn
