// Layout of the per-call scale block in the workspace (zeroed at the start of every
// backward call): det-mode and key-copy scales in its first 16 words, then kKmaxSlots
// words that take the key maximum, one per 128-byte line.
#pragma once

namespace slikl {

constexpr int kKmaxBase = 32;
constexpr int kKmaxSlots = 16;
constexpr int kScaleBlockBytes = 4 * (kKmaxBase + 32 * kKmaxSlots);

}  // namespace slikl
