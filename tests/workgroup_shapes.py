"""The forward's workgroup shapes (query blocks per workgroup G, key slices
KS) as the library instantiates them, for the shape tests.

A shape exists when it is one of INSTANTIATED, has at most 8 waves
((bs / 32) * G * KS) and its LDS ring fits a workgroup.  The five shapes of
REFUSED_LDS are instantiated but need more LDS than a workgroup has (their
ring of two or three K+V buffers, or the key slices' merge area); the library
refuses them with BSA_ERR_INVALID_ARGUMENT before any launch."""

INSTANTIATED = [(1, 1), (1, 2), (1, 4), (2, 1), (4, 1)]
NOT_INSTANTIATED = [(1, 8), (2, 2), (2, 4), (4, 2)]
REFUSED_LDS = {("bf16", 64, 128, 1, 4), ("f32", 32, 128, 1, 4), ("f32", 64, 64, 1, 4),
               ("f32", 64, 128, 1, 2), ("f32", 64, 128, 1, 4)}
CONFIGS = [(dt, bs, d) for dt in ("bf16", "f32") for bs in (32, 64) for d in (64, 128)]


def waves(bs, group, key_split):
    return (bs // 32) * group * key_split


def runnable(dt, bs, d, group, key_split):
    return ((group, key_split) in INSTANTIATED and waves(bs, group, key_split) <= 8
            and (dt, bs, d, group, key_split) not in REFUSED_LDS)


def runnable_cases(configs=CONFIGS):
    """(dt, bs, d, group, key_split) of every shape the library runs."""
    return [(dt, bs, d, g, ks) for dt, bs, d in configs for g, ks in INSTANTIATED
            if runnable(dt, bs, d, g, ks)]


def refused_cases(configs=CONFIGS):
    """Shapes with at most 8 waves that the library must refuse."""
    return [(dt, bs, d, g, ks) for dt, bs, d in configs
            for g, ks in INSTANTIATED + NOT_INSTANTIATED
            if waves(bs, g, ks) <= 8 and not runnable(dt, bs, d, g, ks)]
