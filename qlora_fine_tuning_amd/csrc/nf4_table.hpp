// fp32 bit patterns of the 16 NF4 levels, ascending (level 0 = -1, level 7 =
// exact 0, level 15 = +1). Construction: asymmetric normal-quantile table with
// delta = 31/32; the 8 positive levels are Phi^-1(1/2 + (delta - 1/2) j / 8),
// j = 1..8, the 7 negative levels -Phi^-1(1/2 + (delta - 1/2) j / 7),
// j = 1..7, all divided by Phi^-1(delta) and rounded once to fp32.
#pragma once
#define QLORA_NF4_LEVEL_BITS                                                  \
  0xbf800000u, 0xbf3188d6u, 0xbf05c6b0u, 0xbec92605u, 0xbe90d881u,            \
      0xbe3c28e3u, 0xbdb96cbbu, 0x00000000u, 0x3da210d6u, 0x3e23e03bu,        \
      0x3e7aa402u, 0x3eac17c0u, 0x3ee08015u, 0x3f0f5d29u, 0x3f38654du,        \
      0x3f800000u
