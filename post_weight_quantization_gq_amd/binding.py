"""placeholder; replaced below"""
class GQError(RuntimeError):
    pass
def library(): raise GQError("not built")
abi_version = fisher = lnq_codebook_update = lnq_assign_sweep = lnq_objective = lnq_quantize = lnq_options = library
